// Block selection: normalise the block scores and keep the forced set plus
// the Top-(Kb-3) of the rest.
//
// CompKV page (onedev.kr/papers/157), "What differs": p̂_{g,b} is the
// log-normal mass estimate normalised over all blocks,
//   p̂_{g,b} = |b| exp(z̄ + σ̂²/2) / sum_c |c| exp(z̄_c + σ̂²_c/2),
// S_b = sum_g p̂_{g,b} σ̂²_{g,b}; the first block and the two most recent
// blocks are always kept and count against the budget; the remaining slots
// go to the largest S_b (ties: lower block index).
//
// One 512-thread workgroup per unit (8 waves: barriers stay cheap); thread t
// computes the keys of blocks t + 512*m (coalesced) and, once they have
// passed through LDS, selects on the run of KPT consecutive blocks it then
// owns (KPT the smallest of 2, 4, 6, 8, 12, 17 and 24 that covers
// max_blocks: a larger one only loads and scans empty slots). The
// score kernel left, per 16-block group, the partial (max, sum) of
// a = ln|b| + z̄ + σ̂²/2 per query head and, per block,
// u_{g,b} = exp(a - group max) σ̂². Here:
//   1. LSE_g from the chunk partials (wave g reduces query head g's);
//      S_b = sum_g u_{g,b} exp(group max - LSE_g);
//      the key of a block is the fp32 bit pattern of S_b (S_b >= 0, so keys
//      order like values).
//   2. A 2048-bin histogram of the candidates' (not forced) key top 11 bits;
//      one wave finds the bin B holding the (Kb-3)-th largest key.
//   3. Keys above B are kept. The keys inside B go to a short list that is
//      ordered exactly by (key desc, index asc); its first `krem` are kept.
//      If B holds more than kListMax keys (long runs of equal scores), two
//      more radix passes (11 and 10 bits) pin the exact threshold key instead
//      and equal keys are taken in index order.
//   4. The kept blocks are written in ascending order (one workgroup scan of
//      the per-thread counts of the contiguous runs).
#include "select_core.h"

namespace cknv {

namespace {

constexpr int kSelWaves = kSelThreads / 64;

}  // namespace

template <int G, int KPT>
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectArgs a) {
  static_assert(KPT <= kSelKeysPerThread, "the plan's limit");
  static_assert(G <= kSelWaves, "one wave per query head for the normalisers");
  constexpr int NW = KPT * kSelThreads / 32;  // words of the kept-block bitmap
  constexpr int NGmax = kSelThreads * KPT / kScoreMinGroup;  // score groups, at most
  __shared__ float f[NGmax * G];                 // exp(group max - LSE_g)
  __shared__ float lse_s[G];
  __shared__ __align__(16) int hist[2048];
  __shared__ int cnt[KPT * kSelWaves + 1];
  __shared__ __align__(16) uint64_t plist[kListMax + kListPad];  // pivot-bin (key, index) words
  __shared__ uint32_t keys_l[KPT * kSelThreads];                   // every block's key, block order
  __shared__ uint32_t keep_bits[NW];
  __shared__ int ctl[8];

  const int unit = blockIdx.x, s = unit / a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int MB = a.max_blocks;
  int32_t* sel = a.sel + (size_t)unit * a.Kb;
  const float* grp = a.grp + (size_t)unit * a.NG * G * 2;
  const float* u = a.u + (size_t)unit * MB * G;

  // ---- loads, issued before the context length is known (clamped to max_blocks)
  const int T = a.seq_len[s];
  // wave g < G: query head g's chunk partials, chunk lane + 64k (a chunk
  // covers at least 32 blocks; G <= 8 waves)
  constexpr int CPL = (KPT * kSelThreads / 32 + 63) / 64;
  const int NC = a.C;
  float2 hd[CPL];
  {
    const float2* hp = reinterpret_cast<const float2*>(a.hdr) + (size_t)unit * NC * G + (wave < G ? wave : 0);
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      const int c = lane + 64 * k;
      hd[k] = hp[(size_t)(c < NC ? c : NC - 1) * G];
    }
  }
  constexpr int GPT = (NGmax + kSelThreads - 1) / kSelThreads;  // score groups per thread
  float gr[GPT][G];  // the groups' max of a per query head
#pragma unroll
  for (int k = 0; k < GPT; ++k) {
    const int gi = tid + k * kSelThreads;
    const int gc = gi < a.NG ? gi : a.NG - 1;
    float2 v[G];
    load_pairs<G>(reinterpret_cast<const float2*>(grp) + (size_t)gc * G, v);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      gr[k][g] = v[g].x;
    }
  }
  // blocks of u per thread per batch: all of them up to 4 query heads (one round trip)
  // (8 query heads with 6 or 8 slots: 4 rows a batch, 6 spilled at the
  // 1024-thread register cap)
  constexpr int UB1 = G >= 8 && KPT < 12 ? 4 : 48 / G;
  constexpr int UB0 = UB1 < 4 ? 4 : (UB1 > KPT ? KPT : UB1);
  float ub[UB0][G];
#pragma unroll
  for (int m = 0; m < UB0; ++m) {
    const int b = tid + m * kSelThreads;
    const int bc = b < MB ? b : MB - 1;
    load_row<G>(u + (size_t)bc * G, ub[m]);
  }
  for (int i = tid; i < 2048; i += kSelThreads) hist[i] = 0;
  for (int i = tid; i < NW; i += kSelThreads) keep_bits[i] = 0u;
  if (tid == 0) ctl[3] = 0;  // list length
  if (tid < kListMax + kListPad) plist[tid] = 0ull;

  int NB = (T + kBlock - 1) / kBlock;
  NB = NB < MB ? NB : MB;
  if (NB == 0) {
    if (tid == 0) a.n_sel[unit] = 0;
    return;
  }
  const int NGu = (NB + (1 << a.bpw_shift) - 1) >> a.bpw_shift;
  const int nper = (NB + kSelThreads - 1) / kSelThreads;
  const int Kb = a.Kb;
  const bool all = NB <= Kb;
  int krem = Kb - 3;

  // ---- LSE_g over all blocks (wave g reduces head g's chunk partials),
  // f = exp(group max - LSE_g)
  if (wave < G) {
    float r = -INFINITY;
#pragma unroll
    for (int k = 0; k < CPL; ++k) r = fmaxf(r, lane + 64 * k < NC ? hd[k].x : -INFINITY);
    const float M = group_max<64>(r);
    float l = 0.f;
#pragma unroll
    for (int k = 0; k < CPL; ++k) l += lane + 64 * k < NC ? hd[k].y * rescale(hd[k].x, M) : 0.f;
    const float L = group_sum<64>(l);
    if (lane == 0) lse_s[wave] = M + __logf(L);
  }
  lds_barrier();
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float lse = lse_s[g];
#pragma unroll
    for (int k = 0; k < GPT; ++k)
      if (tid + k * kSelThreads < NGu) f[(tid + k * kSelThreads) * G + g] = __expf(gr[k][g] - lse);
  }
  lds_barrier();

  // ---- S_b, its key, and the histogram of the candidates' key top 11 bits
  uint32_t key[KPT];
  const bool count = !all && krem > 0;
  float* scores = a.scores ? a.scores + (size_t)unit * a.cap_blocks : nullptr;
#pragma unroll
  for (int m0 = 0; m0 < KPT; m0 += UB0) {
    if (m0 > 0 && m0 < nper) {
#pragma unroll
      for (int m = 0; m < UB0; ++m) {
        if (m0 + m >= KPT) break;  // (a last batch shorter than UB0)
        const int b = tid + (m0 + m) * kSelThreads;
        const int bc = b < NB ? b : NB - 1;
        load_row<G>(u + (size_t)bc * G, ub[m]);
      }
    }
#pragma unroll
    for (int m = 0; m < UB0; ++m) {
      if (m0 + m >= KPT) break;
      const int b = tid + (m0 + m) * kSelThreads;
      const int bc = b < NB ? b : NB - 1;
      float S = 0.f;
#pragma unroll
      for (int g = 0; g < G; ++g) S += ub[m][g] * f[(bc >> a.bpw_shift) * G + g];
      key[m0 + m] = (b < NB && S > 0.f) ? __float_as_uint(S) : 0u;
      const bool c = b >= 1 && b <= NB - 3;  // a candidate (not forced, in range)
      if (scores && b < NB) scores[b] = S;
      if (c && count) atomicAdd(&hist[key[m0 + m] >> 21], 1);
    }
  }
  if (all) {
    for (int b = tid; b < NB; b += kSelThreads) sel[b] = b;
    if (tid == 0) a.n_sel[unit] = NB;
    return;
  }

  // ---- the keys go through LDS so that from here on thread t holds the run
  // of KPT consecutive blocks b0 = t*KPT ..: block order is thread order, and
  // the list, the tie ranks and the compaction are per-thread counts and one
  // scan instead of a pass per block slot
#pragma unroll
  for (int m = 0; m < KPT; ++m) keys_l[tid + m * kSelThreads] = key[m];
  lds_barrier();  // also completes the histogram
  const int b0 = tid * KPT;
  uint32_t kr[KPT];  // keys of the thread's run
#pragma unroll
  for (int i = 0; i < KPT; ++i) kr[i] = keys_l[b0 + i];
  uint64_t cand = 0u;  // bit i: block b0 + i is a candidate (not forced, in range)
#pragma unroll
  for (int i = 0; i < KPT; ++i) cand |= (uint64_t)(b0 + i >= 1 && b0 + i <= NB - 3) << i;

  // ---- threshold bin: keys whose top 11 bits exceed tau_bin are kept
  uint32_t tau_bin = 0xffffffffu;
  bool use_list = true;
  if (krem > 0) {
    if (wave == 0) find_bin<2048>(hist, krem, ctl);
    lds_barrier();
    tau_bin = (uint32_t)ctl[0];
    krem = ctl[1];
    use_list = ctl[2] <= kListMax;
  }

  uint32_t exact_tau = 0u;  // long-tie path: exact threshold key, ties by index
  uint64_t pin = 0u, gtm = 0u;  // candidates in the pivot bin / in higher bins
  if (krem > 0 && use_list) {
    // the pivot bin's keys, ordered exactly; the first krem are kept
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const bool c = (cand >> i) & 1u;
      const uint32_t kb = kr[i] >> 21;
      pin |= (uint64_t)(c && kb == tau_bin) << i;
      gtm |= (uint64_t)(c && kb > tau_bin) << i;
    }
    run_append(pin, keys_l, b0, plist, &ctl[3]);
    lds_barrier();
    rank_list_keep<kSelThreads>(plist, ctl[3], krem, keep_bits);
    lds_barrier();
  } else if (krem > 0) {
    uint32_t prefix = tau_bin << 21;
    // bits 20..10 among the keys of the pivot bin
    for (int i = tid; i < 2048; i += kSelThreads) hist[i] = 0;
    lds_barrier();
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      if (((cand >> i) & 1u) && (kr[i] >> 21) == (prefix >> 21)) atomicAdd(&hist[(kr[i] >> 10) & 2047u], 1);
    lds_barrier();
    if (wave == 0) find_bin<2048>(hist, krem, ctl);
    lds_barrier();
    prefix |= ((uint32_t)ctl[0]) << 10;
    krem = ctl[1];
    // bits 9..0
    for (int i = tid; i < 1024; i += kSelThreads) hist[i] = 0;
    lds_barrier();
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      if (((cand >> i) & 1u) && (kr[i] >> 10) == (prefix >> 10)) atomicAdd(&hist[kr[i] & 1023u], 1);
    lds_barrier();
    if (wave == 0) find_bin<1024>(hist, krem, ctl);
    lds_barrier();
    prefix |= (uint32_t)ctl[0];
    krem = ctl[1];
    exact_tau = prefix;
  }

  // ---- ascending compaction of the kept blocks
  uint64_t forced = 0u, above = 0u;
  const int fbl[3] = {0, NB - 2, NB - 1};
#pragma unroll
  for (int k = 0; k < 3; ++k)
    if (fbl[k] >= 0 && fbl[k] / KPT == tid) forced |= 1ull << (fbl[k] - b0);
  if (krem > 0 && !use_list) {
    // keys equal to the threshold key are kept in index order: the first krem of them
    uint64_t eqm = 0u;
#pragma unroll
    for (int i = 0; i < KPT; ++i) eqm |= (uint64_t)(((cand >> i) & 1u) && kr[i] == exact_tau) << i;
    int tot;
    const int eq0 = block_excl_scan<kSelWaves>(__popcll(eqm), cnt, tot);
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const bool c = (cand >> i) & 1u;
      const int eb = eq0 + __popcll(eqm & ((1ull << i) - 1ull));
      above |= (uint64_t)(c && (kr[i] > exact_tau || (kr[i] == exact_tau && eb < krem))) << i;
    }
    lds_barrier();  // cnt is scanned again below
  } else if (krem > 0) {
    // every candidate of a higher bin, and the pivot-bin keys the rank kept
    uint64_t kp = 0u;
    for (uint64_t m = pin; m; m &= m - 1) {
      const int i = __builtin_ctzll(m);
      const int b = b0 + i;
      kp |= (uint64_t)((keep_bits[b >> 5] >> (b & 31)) & 1u) << i;
    }
    above = gtm | kp;
  }
  const uint64_t takem = forced | above;
  int nk;
  int pos = block_excl_scan<kSelWaves>(__popcll(takem), cnt, nk);
  for (uint64_t m = takem; m; m &= m - 1, ++pos)
    if (pos < Kb) sel[pos] = b0 + __builtin_ctzll(m);
  if (tid == 0) a.n_sel[unit] = Kb;
}

hipError_t launch_select(int G, const SelectArgs& a, int U, hipStream_t st) {
  void* args[] = {(void*)&a};
  const int mb = a.max_blocks;
  const int kpt = mb <= 2 * kSelThreads ? 2 : mb <= 4 * kSelThreads ? 4 : mb <= 6 * kSelThreads ? 6
                : mb <= 8 * kSelThreads ? 8 : mb <= 12 * kSelThreads ? 12 : mb <= 17 * kSelThreads ? 17 : 24;
  const void* f = nullptr;
#define CKNV_SEL_G(GG)                                                                          \
  if (G == GG)                                                                                  \
    f = kpt == 2 ? (const void*)select_kernel<GG, 2> : kpt == 4 ? (const void*)select_kernel<GG, 4> \
      : kpt == 6 ? (const void*)select_kernel<GG, 6> : kpt == 8 ? (const void*)select_kernel<GG, 8> \
      : kpt == 12 ? (const void*)select_kernel<GG, 12> : kpt == 17 ? (const void*)select_kernel<GG, 17> \
                  : (const void*)select_kernel<GG, 24>;
  CKNV_SEL_G(1) CKNV_SEL_G(2) CKNV_SEL_G(4) CKNV_SEL_G(8)
#undef CKNV_SEL_G
  if (!f || mb > kSelThreads * kSelKeysPerThread) return hipErrorInvalidValue;
  return hipLaunchKernel(f, dim3(U), dim3(kSelThreads), args, 0, st);
}

}  // namespace cknv
