// Block scoring: one streaming pass over the summary store.
//
// CompKV page (onedev.kr/papers/157), "What differs": for the G query heads
// of a KV head and every block b,
//   z̄_{g,b}  = q_g . k̄_b / sqrt(d)
//   σ̂²_{g,b} = (1/d) sum_t (sum_{i in G_t} q_{g,i}^2) D̄_{b,t}
//   p̂_{g,b}  = |b| exp(z̄ + σ̂²/2) / sum_c |c| exp(z̄_c + σ̂²_c/2)
//   S_b      = sum_g p̂_{g,b} σ̂²_{g,b}
// and the kept set is the first block, the two most recent blocks and the
// Top-(Kb-3) of the rest by S_b. "How it works": an unselected block is
// represented by Mean compensation, |b| e^{z̄} with mean value v̄_b.
// This file computes every block's score ingredients in one streaming pass.
//
// σ̂² is evaluated per coordinate, (1/d) sum_i q_{g,i}^2 D̄_{b,t(i)} with t(i)
// the group of coordinate i, which is the same sum regrouped.
//
// Grid: C workgroups ("chunks") per unit of kScoreWaves waves, 4*ROWS blocks
// per wave; a block is read by 16 lanes (d/64 float4 of k̄, D̄ and v̄ each), so
// the wave reads 4 blocks' rows per load instruction. For one sequence every
// load is issued before seq_len is known (max_blocks bounds the block index);
// a batch of several waits for it, so that a short sequence's chunks past its
// end re-read one row instead of unused summaries. Blocks past the context
// are masked afterwards. Per wave
// (a 16-block group) the kernel writes the LSE partial of
// a = ln|b| + z̄ + σ̂²/2 and per block u_{g,b} = exp(a - group max) σ̂²; per
// chunk it writes the Mean-compensation sums of ALL its blocks,
//   (m, l = sum |b| e^{z̄-m}, acc = sum |b| e^{z̄-m} v̄_b),
// which the attend kernel corrects by removing the kept blocks' terms (the
// kept set is not known yet), and apart from it the chunk's LSE partial of a
// per query head. The selection kernel (select.hip) runs next.
//
// In the fused step the grid starts with one extra workgroup per unit that
// appends the step's token and summarises the block it lands in ("How to use
// it": the current block's statistics are refreshed every step); the
// scoring workgroups then cover only the blocks closed before the token.
#include "cknv_internal.h"
#include "summary_core.h"

namespace cknv {

namespace {

// How σ̂² is formed. kDbarRow (r <= 8): per (block, head) from the block's r
// D̄ entries and the head's r group energies E_t = sum_{i in G_t} q_i^2, the
// page's form; kDbarRow4 is the same for r = 4, the block's D̄ in one 16-byte
// load. Otherwise per coordinate and summed over the block's lanes with z̄;
// then how a lane's 4 coordinates 4c..4c+3 map to D̄ entries (group size
// gs = d/r).
enum DbarMode { kDbarOne = 0, kDbarPair = 1, kDbarQuad = 2, kDbarRow = 3, kDbarRow4 = 4 };  // gs >= 4, gs == 2, gs == 1; r <= 8; r == 4
constexpr int kRowMaxR = 8;
constexpr bool row_mode(int dm) { return dm == kDbarRow || dm == kDbarRow4; }

__device__ __forceinline__ float dot4(const float4 a, const float4 b) {
  return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}

// D̄ entries of a lane's coordinates, stored at their natural width, and
// sum_e q_e^2 D̄_{t(4c+e)} over the lane's 4 coordinates of chunk c.
template <int DM, int ROWS, int KC>
struct DbarTile;
template <int ROWS, int KC>
struct DbarTile<kDbarOne, ROWS, KC> {
  float x[ROWS][KC];
  __device__ void load(const float* dbar, size_t row, int c, int r, int D, int rw, int i) {
    x[rw][i] = dbar[row * r + (4 * c) / (D / r)];
  }
  __device__ float qsq_dot(const float4 q, int rw, int i) const {
    return (q.x * q.x + q.y * q.y + q.z * q.z + q.w * q.w) * x[rw][i];
  }
};
template <int ROWS, int KC>
struct DbarTile<kDbarPair, ROWS, KC> {
  float2 x[ROWS][KC];
  __device__ void load(const float* dbar, size_t row, int c, int r, int D, int rw, int i) {
    x[rw][i] = reinterpret_cast<const float2*>(dbar)[row * (D / 4) + c];
  }
  __device__ float qsq_dot(const float4 q, int rw, int i) const {
    return (q.x * q.x + q.y * q.y) * x[rw][i].x + (q.z * q.z + q.w * q.w) * x[rw][i].y;
  }
};
template <int ROWS, int KC>
struct DbarTile<kDbarRow, ROWS, KC> {  // unused: σ̂² is formed per (block, head)
  __device__ void load(const float*, size_t, int, int, int, int, int) {}
  __device__ float qsq_dot(const float4, int, int) const { return 0.f; }
};
template <int ROWS, int KC>
struct DbarTile<kDbarRow4, ROWS, KC> : DbarTile<kDbarRow, ROWS, KC> {};
template <int ROWS, int KC>
struct DbarTile<kDbarQuad, ROWS, KC> {
  float4 x[ROWS][KC];
  __device__ void load(const float* dbar, size_t row, int c, int r, int D, int rw, int i) {
    x[rw][i] = reinterpret_cast<const float4*>(dbar)[row * (D / 4) + c];
  }
  __device__ float qsq_dot(const float4 q, int rw, int i) const {
    const float4 d = x[rw][i];
    return q.x * q.x * d.x + q.y * q.y * d.y + q.z * q.z * d.z + q.w * q.w * d.w;
  }
};

}  // namespace

// Partner across lane bit K (distance 2^K) inside a 16-lane row.
template <int K>
__device__ __forceinline__ float xlane(float x) {
  if constexpr (K == 0) return dpp<kDppXor1>(x);
  else if constexpr (K == 1) return dpp<kDppXor2>(x);
  else if constexpr (K == 2) return dpp<kDppQuadRev>(dpp<kDppHalfMirror>(x));  // xor 7, then xor 3
  else return dpp<kDppRor8>(x);
}

// One butterfly step over lane bit K on x[0..N): plain (every lane sums
// every value with its partner) or transposed (pairs x[m], x[m+N/2]; lanes
// with bit K clear keep the sum of the lower one, lanes with it set the
// upper one, so the count halves).
template <int K, int N, int CAP>
__device__ __forceinline__ void plain_step(float (&x)[CAP]) {
#pragma unroll
  for (int m = 0; m < N; ++m) x[m] += xlane<K>(x[m]);
}
template <int K, int N, int CAP>
__device__ __forceinline__ void transposed_step(float (&x)[CAP], bool hi) {
#pragma unroll
  for (int m = 0; m < N / 2; ++m) {
    const float A = x[m], B = x[m + N / 2];
    x[m] = (hi ? B : A) + xlane<K>(hi ? A : B);
  }
}

// Sum over the 16 lanes of each row of 2*NP values per lane, value index
// p + 2*i (p in {0,1}, i < NP). Afterwards x[0], x[1] of lane j hold the sums
// for i = j & (NP-1).
template <int NP, int CAP>
__device__ __forceinline__ void reduce_rows16(float (&x)[CAP], int j) {
  constexpr int N = 2 * NP;
  if constexpr (NP < 16) plain_step<3, N>(x);
  if constexpr (NP < 8) plain_step<2, N>(x);
  if constexpr (NP < 4) plain_step<1, N>(x);
  if constexpr (NP >= 16) transposed_step<3, N>(x, (j & 8) != 0);
  if constexpr (NP >= 8) transposed_step<2, (NP >= 16 ? N / 2 : N)>(x, (j & 4) != 0);
  if constexpr (NP >= 4) transposed_step<1, (NP >= 16 ? N / 4 : NP >= 8 ? N / 2 : N)>(x, (j & 2) != 0);
  transposed_step<0, 4>(x, (j & 1) != 0);
}

// Sum over the 16 lanes of each row of NP values per lane (value index i <
// NP). Afterwards x[0] of lane j holds the sum for i = j & (NP-1).
template <int NP, int CAP>
__device__ __forceinline__ void reduce_rows16_1(float (&x)[CAP]) {
  const int j = threadIdx.x & 15;
  if constexpr (NP < 16) plain_step<3, NP>(x);
  if constexpr (NP < 8) plain_step<2, NP>(x);
  if constexpr (NP < 4) plain_step<1, NP>(x);
  if constexpr (NP < 2) plain_step<0, NP>(x);
  if constexpr (NP >= 16) transposed_step<3, 16>(x, (j & 8) != 0);
  if constexpr (NP >= 8) transposed_step<2, 8>(x, (j & 4) != 0);
  if constexpr (NP >= 4) transposed_step<1, 4>(x, (j & 2) != 0);
  if constexpr (NP >= 2) transposed_step<0, 2>(x, (j & 1) != 0);
}

// Max / sum over the SEG consecutive lanes (SEG = 2 or 4) of each aligned segment.
template <int SEG>
__device__ __forceinline__ float seg_max(float x) {
  x = fmaxf(x, dpp<kDppXor1>(x));
  if constexpr (SEG >= 4) x = fmaxf(x, dpp<kDppXor2>(x));
  return x;
}
template <int SEG>
__device__ __forceinline__ float seg_sum(float x) {
  x += dpp<kDppXor1>(x);
  if constexpr (SEG >= 4) x += dpp<kDppXor2>(x);
  return x;
}

template <int L>
__device__ __forceinline__ float row_bcast(float x) { return dpp<kDppBcast0 + L>(x); }

// Fused step, wave 0 of workgroup `unit`: store the token (new_k, new_v) at
// slot T0 = seq_len, summarise its block from the np = T0 % 16 cached tokens
// and the new one ({|b|, k̄, D̄, v̄}, population variances, D̄ over contiguous
// groups of d/r coordinates), and write that block's a and its factor in S
// (σ̂², or 1 for the mass-only ablation) per query head to finfo. A sequence
// whose cache is full (or whose block lies past max_blocks) appends nothing
// and gets a = -inf. Lane l owns coordinates [l*VPL, l*VPL + VPL).
template <int D, int G>
__device__ void fresh_block(const ScoreArgs& a, int unit) {
  constexpr int VPL = D / 64;
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  const int s = unit / a.H, h = unit - s * a.H;
  const int T0 = a.seq_len[s];
  const long cap_tok = (long)a.cap_blocks * kBlock;
  const int fblk = T0 / kBlock;
  const bool app = T0 < cap_tok && fblk < a.max_blocks;
  float2* fi = reinterpret_cast<float2*>(a.finfo) + (size_t)unit * G;
  for (int i = lane; i < a.pstride; i += 64) a.pcnt[(size_t)unit * a.pstride + i] = 0u;  // read by the step kernel
  if (!app) {
    if (lane < G) fi[lane] = make_float2(-INFINITY, 0.f);
    if (h == 0 && lane == 0) a.t0_out[s] = T0;
    return;
  }
  uint16_t* kc = a.k + (size_t)unit * cap_tok * D;
  uint16_t* vc = a.v + (size_t)unit * cap_tok * D;
  const long tok0 = (long)fblk * kBlock;
  const int np = T0 - fblk * kBlock, n = np + 1;
  uint32_t fk[16], fv[16];
  load_block_words<D, false>(kc, vc, tok0, np, lane, fk, fv);  // the np cached tokens
  const size_t noff = (size_t)unit * D + lane * VPL;
  const uint32_t nkw = VPL == 2 ? *reinterpret_cast<const uint32_t*>(a.new_k + noff) : (uint32_t)a.new_k[noff];
  const uint32_t nvw = VPL == 2 ? *reinterpret_cast<const uint32_t*>(a.new_v + noff) : (uint32_t)a.new_v[noff];
  float fq[G][VPL];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < VPL; ++e) fq[g][e] = a.q[((size_t)unit * G + g) * D + lane * VPL + e];
#pragma unroll
  for (int j = 0; j < 16; ++j) {  // the new token is token np
    fk[j] = j < np ? fk[j] : nkw;
    fv[j] = j < np ? fv[j] : nvw;
  }
  float km[VPL], vm[VPL], dl[VPL];
  block_summary<D>(fk, fv, n, a.r, km, vm, dl);
  const float half = (a.flags & CKNV_FLAG_FIRST_ORDER_MASS) ? 0.f : 0.5f;
  const bool mass_only = (a.flags & CKNV_FLAG_MASS_ONLY_SCORE) != 0;
  float2 info = make_float2(-INFINITY, 0.f);
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
    if (lane == g) info = make_float2(__logf((float)n) + z + half * s2, mass_only ? 1.f : s2);
  }
  // every store after the last load
  if (lane < G) fi[lane] = info;
  const size_t toff = (size_t)T0 * D + lane * VPL;
  const size_t row = (size_t)unit * a.cap_blocks + fblk;
  if (VPL == 2) {
    *reinterpret_cast<uint32_t*>(kc + toff) = nkw;
    *reinterpret_cast<uint32_t*>(vc + toff) = nvw;
  } else {
    kc[toff] = (uint16_t)nkw;
    vc[toff] = (uint16_t)nvw;
  }
  store_block_summary<D>(a.kbar, a.dbar, a.cnt, a.vbar, row, a.r, n, lane, km, vm, dl);
  if (h == 0 && lane == 0) a.t0_out[s] = T0;
}

// Deferred mean values: at 4 query heads with σ̂² per (block, head), v̄ is
// loaded once z̄ and σ̂² are formed. The first loads (k̄, D̄, |b|) then return
// sooner, and the v̄ loads overlap the scoring partials (measured faster at
// 32K and 128K). At 4 rows k̄ and v̄ are never live together, so 5 waves fit
// per SIMD: a grid of 4096 scoring waves plus the append workgroups is then
// resident in one round on 256 CUs.
template <int G, int DM, int ROWS, bool NC>
constexpr bool score_defers_vbar() { return !NC && row_mode(DM) && G == 4; }
template <int G, int DM, int ROWS, bool NC>
constexpr int score_waves_per_simd() { return score_defers_vbar<G, DM, ROWS, NC>() && ROWS == 4 ? 5 : 1; }

// NC: the no-compensation ablation; the mean values are neither read nor summed.
// ONE: a batch of one sequence (the loads do not wait for seq_len).
template <int D, int G, int DM, int ROWS, bool NC, bool ONE>
__global__ __launch_bounds__(kScoreThreads)
__attribute__((amdgpu_waves_per_eu(score_waves_per_simd<G, DM, ROWS, NC>())))
void score_kernel(ScoreArgs a) {
  constexpr int KC = D / 64;              // float4 chunks per lane per block (16 lanes per block)
  constexpr bool kDeferV = score_defers_vbar<G, DM, ROWS, NC>();
  constexpr int E = 4 * KC;               // coordinates per lane
  // ROWS: blocks per lane, base + 4*row + (lane >> 4)
  constexpr int NP = ROWS * G;            // (row, head) pairs of a 16-lane row
  constexpr int BPW = 4 * ROWS, BPWG = kScoreWaves * BPW;
  constexpr int W = rec_words(D);
  constexpr int NA = G * E;               // compensation sums per lane before the cross-row step
  __shared__ __align__(16) float cacc[kScoreWaves * G * D];  // per-wave compensation sums
  __shared__ float cml[kScoreWaves * G * 2];                 // per-wave (max, normaliser) of z̄
  __shared__ float cma[kScoreWaves * G * 2];                 // per-wave (max, normaliser) of a
  __shared__ __align__(16) float4 q_s[G * D / 4];            // the G query heads
  __shared__ float e_s[G * kRowMaxR];                        // row modes: group energies E[g][t]

  // The scoring path's kernel arguments are read with the first batch: used
  // only after the branch below, their loads would otherwise be issued (and
  // waited for) there, one more round trip before the first summary load.
  asm volatile("" ::"s"(a.NG), "s"(a.C), "s"(a.xcd), "s"(a.rows));
  if ((int)blockIdx.x < a.nfresh) {
    fresh_block<D, G>(a, blockIdx.x);
    return;
  }
  int unit, chunk;
  map_wg(blockIdx.x - a.nfresh, a.S * a.H, a.C, a.xcd, unit, chunk);
  const int s = unit / a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bg = lane >> 4, j = lane & 15;
  const int r = a.r, MB = a.max_blocks;
  const int base = chunk * BPWG + wave * BPW;
  const size_t ubase = (size_t)unit * a.cap_blocks;
  // After the transposed reduction this lane holds block tb, query head tg.
  const int pj = j & (NP - 1);
  const int trow = pj % ROWS, tg = pj / ROWS;
  const int tb = base + 4 * trow + bg;

  // ---- every load of the workgroup, issued before any result is needed.
  // Block indices are clamped into [0, MB); blocks past the scored range are
  // masked once seq_len has arrived.
  // the query goes to LDS (registers are what limits resident waves here)
  static_assert(G * D / 4 <= kScoreThreads, "one float4 of q per thread");
  const float4 qown = reinterpret_cast<const float4*>(a.q + (size_t)unit * G * D)[tid < G * D / 4 ? tid : 0];
  float4 kv[ROWS][KC], vv[ROWS][KC];
  DbarTile<DM, ROWS, KC> dt;
  float n;
  float dbr[kRowMaxR];  // kDbarRow, kDbarRow4: D̄ of this lane's block tb
  const float4* kbar4 = reinterpret_cast<const float4*>(a.kbar);
  const float4* vbar4 = reinterpret_cast<const float4*>(a.vbar);
  // lim: the highest block index read (indices are clamped to it)
  auto issue_loads = [&](int lim) {
#pragma unroll
    for (int rw = 0; rw < ROWS; ++rw) {
      const int b = base + 4 * rw + bg;
      const size_t row = ubase + (b < lim ? b : lim);
#pragma unroll
      for (int i = 0; i < KC; ++i) {
        const int c = j + 16 * i;  // float4 chunk: coordinates 4c..4c+3
        kv[rw][i] = stream_load4(kbar4 + row * (D / 4) + c);
        if constexpr (!NC && !kDeferV) vv[rw][i] = stream_load4(vbar4 + row * (D / 4) + c);
        dt.load(a.dbar, row, c, r, D, rw, i);
      }
    }
    const size_t trow_idx = ubase + (tb < lim ? tb : lim);
    n = a.cnt[trow_idx];
    if constexpr (DM == kDbarRow4) {
      const float4 d4 = *reinterpret_cast<const float4*>(a.dbar + trow_idx * 4);
      dbr[0] = d4.x; dbr[1] = d4.y; dbr[2] = d4.z; dbr[3] = d4.w;
    } else if constexpr (DM == kDbarRow) {
#pragma unroll
      for (int t = 0; t < kRowMaxR; ++t) dbr[t] = a.dbar[trow_idx * r + (t < r ? t : r - 1)];  // masked at use
    }
  };
  // One sequence: the addresses do not wait for seq_len (max_blocks bounds
  // it), which is read after the loads are issued. A batch of several: a
  // chunk past its sequence's end reads one row again and again (cached)
  // instead of max_blocks' worth of unused rows. (Two kernel instances: a
  // run-time branch between the two made the loads wait for seq_len.)
  auto blocks_of = [&](int T) {
    const int nb = a.closed_only ? T / kBlock : (T + kBlock - 1) / kBlock;
    return nb < MB ? nb : MB;
  };
  int T, NB, lim;
  if constexpr (ONE) {
    issue_loads(MB - 1);
    lim = MB - 1;
  } else {
    T = a.seq_len[s];
    NB = blocks_of(T);
    if (chunk * BPWG >= NB) {
      // The whole chunk lies past this sequence's end (a shorter sequence of
      // the batch): an empty header and an empty compensation record, no
      // loads. Its groups and u terms are never read.
      if (tid < G)
        reinterpret_cast<float2*>(a.hdr)[((size_t)unit * a.C + chunk) * G + tid] = make_float2(-INFINITY, 0.f);
      if constexpr (!NC) {
        float* co = a.comp + ((size_t)unit * a.C + chunk) * G * W;
        for (int i = tid; i < G * W; i += kScoreThreads) co[i] = i % W == 0 ? -INFINITY : 0.f;
      }
      return;
    }
    lim = NB - 1;
    issue_loads(lim);
  }
  // Keep the load block above: without this the scheduler sinks loads next
  // to their uses and the wave pays several dependent memory round trips.
  __builtin_amdgcn_sched_barrier(0);
  if (tid < G * D / 4) q_s[tid] = qown;
  lds_barrier();
  if constexpr (row_mode(DM)) {
    // E[g][t]: thread g*r + t sums its group's squared coordinates
    if (tid < G * r) {
      const int g = tid / r, t = tid - g * r, gs4 = D / r / 4;
      const float4* qg = q_s + g * (D / 4) + t * gs4;
      float e = 0.f;
      for (int c = 0; c < gs4; ++c) e += qg[c].x * qg[c].x + qg[c].y * qg[c].y + qg[c].z * qg[c].z + qg[c].w * qg[c].w;
      e_s[g * kRowMaxR + t] = e;
    }
    lds_barrier();
  }
  if constexpr (ONE) {
    // seq_len is read after the query is staged: it is the last load issued,
    // so waiting for it waits for every summary load, and the staging and
    // the group energies above then run while the summaries are in flight
    T = a.seq_len[s];
    NB = blocks_of(T);
  }

  const float invd = 1.0f / (float)D;

  // ---- z̄ (and, per coordinate, σ̂²) partials over the lane's coordinates for
  // every (row, head), then summed over the block's 16 lanes, transposed: lane
  // j ends with (tb, tg).
  float z, s2;
  if constexpr (row_mode(DM)) {
    float x[NP];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float4 qg[KC];
#pragma unroll
      for (int i = 0; i < KC; ++i) qg[i] = q_s[g * (D / 4) + j + 16 * i];
#pragma unroll
      for (int rw = 0; rw < ROWS; ++rw) {
        float zp = 0.f;
#pragma unroll
        for (int i = 0; i < KC; ++i) zp += dot4(kv[rw][i], qg[i]);
        x[rw + ROWS * g] = zp;
      }
    }
    reduce_rows16_1<NP>(x);
    z = x[0] * a.isd;
    float sp = 0.f;
#pragma unroll
    for (int t = 0; t < (DM == kDbarRow4 ? 4 : kRowMaxR); ++t)
      sp += (DM == kDbarRow4 || t < r) ? e_s[tg * kRowMaxR + t] * dbr[t] : 0.f;
    s2 = sp * invd;
  } else {
    float x[2 * NP];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float4 qg[KC];
#pragma unroll
      for (int i = 0; i < KC; ++i) qg[i] = q_s[g * (D / 4) + j + 16 * i];
#pragma unroll
      for (int rw = 0; rw < ROWS; ++rw) {
        float zp = 0.f, sp = 0.f;
#pragma unroll
        for (int i = 0; i < KC; ++i) {
          zp += dot4(kv[rw][i], qg[i]);
          sp += dt.qsq_dot(qg[i], rw, i);
        }
        x[2 * (rw + ROWS * g)] = zp;
        x[2 * (rw + ROWS * g) + 1] = sp;
      }
    }
    reduce_rows16<NP>(x, j);
    z = x[0] * a.isd;
    s2 = x[1] * invd;
  }
  if constexpr (kDeferV) {
#pragma unroll
    for (int rw = 0; rw < ROWS; ++rw) {
      const int b = base + 4 * rw + bg;
      const size_t row = ubase + (b < lim ? b : lim);
#pragma unroll
      for (int i = 0; i < KC; ++i) vv[rw][i] = stream_load4(vbar4 + row * (D / 4) + j + 16 * i);
    }
  }
  const bool tv = tb < NB && j < NP;  // a valid block, and not a duplicate lane (NP < 16)

  // ---- scoring partials of this wave's group: a = ln|b| + z̄ + σ̂²/2, and
  // u = e^{a - group max} σ̂². The first-order-mass ablation drops σ̂²/2 from a,
  // the mass-only ablation drops the factor σ̂² from u.
  const float half = (a.flags & CKNV_FLAG_FIRST_ORDER_MASS) ? 0.f : 0.5f;
  const float av = tv ? __logf(n) + z + half * s2 : -INFINITY;
  const float aref = rows_max(seg_max<ROWS>(av));
  const float ae = tv ? __expf(av - aref) : 0.f;
  const float al = rows_sum(seg_sum<ROWS>(ae));
  {
    const float uf = (a.flags & CKNV_FLAG_MASS_ONLY_SCORE) ? 1.f : s2;
    if (tv) a.u[((size_t)unit * MB + tb) * G + tg] = ae * uf;
    if (base < NB && lane < NP && trow == 0)
      reinterpret_cast<float2*>(a.grp)[((size_t)unit * a.NG + base / BPW) * G + tg] = make_float2(aref, al);
  }
  const bool head_lane = bg == 0 && lane < NP && trow == 0;  // one lane per query head tg
  if (head_lane) {
    cma[(wave * G + tg) * 2] = aref;
    cma[(wave * G + tg) * 2 + 1] = al;
  }
  if constexpr (NC) {
    // no compensation: the record carries only the chunk's LSE partial of a
    lds_barrier();
    if (tid < G) {
      float M = -INFINITY;
#pragma unroll
      for (int q = 0; q < kScoreWaves; ++q) M = fmaxf(M, cma[(q * G + tid) * 2]);
      float L = 0.f;
#pragma unroll
      for (int q = 0; q < kScoreWaves; ++q) L += cma[(q * G + tid) * 2 + 1] * rescale(cma[(q * G + tid) * 2], M);
      reinterpret_cast<float2*>(a.hdr)[((size_t)unit * a.C + chunk) * G + tid] = make_float2(M, L);
    }
    return;
  }

  // ---- Mean compensation of every block of the wave (kept ones are removed later)
  const float mz = rows_max(seg_max<ROWS>(tv ? z : -INFINITY));
  const float w = tv ? n * __expf(z - mz) : 0.f;
  const float lz = rows_sum(seg_sum<ROWS>(w));
  float y[NA];
#pragma unroll
  for (int m = 0; m < NA; ++m) y[m] = 0.f;
#pragma unroll
  for (int rw = 0; rw < ROWS; ++rw) {
    const bool rv = base + 4 * rw + bg < NB;  // the mean value of an unscored block may be anything
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float wb;
      // w of (row rw, head g) lives in lane rw + ROWS*g of this 16-lane row
#define CKNV_BC(L) case L: wb = row_bcast<(L < NP ? L : 0)>(w); break;
      switch (rw + ROWS * g) {
        CKNV_BC(0) CKNV_BC(1) CKNV_BC(2) CKNV_BC(3) CKNV_BC(4) CKNV_BC(5) CKNV_BC(6) CKNV_BC(7)
        CKNV_BC(8) CKNV_BC(9) CKNV_BC(10) CKNV_BC(11) CKNV_BC(12) CKNV_BC(13) CKNV_BC(14) CKNV_BC(15)
        default: wb = 0.f;
      }
#undef CKNV_BC
#pragma unroll
      for (int i = 0; i < KC; ++i) {
        const float4 v4 = vv[rw][i];
        y[g * E + 4 * i + 0] += wb * (rv ? v4.x : 0.f);
        y[g * E + 4 * i + 1] += wb * (rv ? v4.y : 0.f);
        y[g * E + 4 * i + 2] += wb * (rv ? v4.z : 0.f);
        y[g * E + 4 * i + 3] += wb * (rv ? v4.w : 0.f);
      }
    }
  }
  // Sum over the 4 rows of the wave, transposed: rows keep NA/4 values each.
#pragma unroll
  for (int m = 0; m < NA / 2; ++m) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(y[m]), __float_as_uint(y[m + NA / 2]), false, false);
    y[m] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  }
#pragma unroll
  for (int m = 0; m < NA / 4; ++m) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(y[m]), __float_as_uint(y[m + NA / 4]), false, false);
    y[m] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  }
  // Value m of this lane is index v = (bg&1)*NA/2 + (bg>>1)*NA/4 + m = g*E + e.
  {
    const int v0 = (bg & 1) * (NA / 2) + (bg >> 1) * (NA / 4);
    float* cw = cacc + wave * G * D;
#pragma unroll
    for (int m = 0; m < NA / 4; ++m) {
      const int v = v0 + m, g = v / E, e = v % E;
      cw[g * D + 4 * (j + 16 * (e / 4)) + (e % 4)] = y[m];
    }
    if (head_lane) {
      cml[(wave * G + tg) * 2] = mz;
      cml[(wave * G + tg) * 2 + 1] = lz;
    }
  }
  lds_barrier();
  // ---- the workgroup's record: the waves' sums under their common max
  constexpr int CPT = (G * D + kScoreThreads - 1) / kScoreThreads;  // coordinates per thread (1, 2 or 4)
  const int f0 = tid * CPT;
  if (f0 < G * D) {
    const int g = f0 / D, c0 = f0 - g * D;
    float mw[kScoreWaves], M = -INFINITY;
#pragma unroll
    for (int q = 0; q < kScoreWaves; ++q) { mw[q] = cml[(q * G + g) * 2]; M = fmaxf(M, mw[q]); }
    float sc[kScoreWaves];
#pragma unroll
    for (int q = 0; q < kScoreWaves; ++q) sc[q] = rescale(mw[q], M);
    float acc[CPT];
#pragma unroll
    for (int e = 0; e < CPT; ++e) acc[e] = 0.f;
#pragma unroll
    for (int q = 0; q < kScoreWaves; ++q)
#pragma unroll
      for (int e = 0; e < CPT; ++e) acc[e] += cacc[(q * G + g) * D + c0 + e] * sc[q];
    float* co = a.comp + (((size_t)unit * a.C + chunk) * G + g) * W;
#pragma unroll
    for (int e = 0; e < CPT; ++e) co[4 + c0 + e] = acc[e];
    if (c0 == 0) {
      float l = 0.f;
#pragma unroll
      for (int q = 0; q < kScoreWaves; ++q) l += cml[(q * G + g) * 2 + 1] * sc[q];
      float Ma = -INFINITY, La = 0.f;
#pragma unroll
      for (int q = 0; q < kScoreWaves; ++q) Ma = fmaxf(Ma, cma[(q * G + g) * 2]);
#pragma unroll
      for (int q = 0; q < kScoreWaves; ++q) La += cma[(q * G + g) * 2 + 1] * rescale(cma[(q * G + g) * 2], Ma);
      *reinterpret_cast<float2*>(co) = make_float2(M, l);
      reinterpret_cast<float2*>(a.hdr)[((size_t)unit * a.C + chunk) * G + g] = make_float2(Ma, La);
    }
  }
}

hipError_t launch_score(int d, int G, const ScoreArgs& a, int U, hipStream_t st) {
  void* args[] = {(void*)&a};
  const int gs = d / a.r;
  const int dm = a.r == 4 ? kDbarRow4 : a.r <= kRowMaxR ? kDbarRow : gs >= 4 ? kDbarOne : (gs == 2 ? kDbarPair : kDbarQuad);
  const void* f = nullptr;
  const bool nc = (a.flags & CKNV_FLAG_NO_COMPENSATION) != 0;
  const bool one = a.S == 1;
#define CKNV_SCORE_ONE(DD, GG, RR, NC, ONE)                                       \
  f = dm == kDbarRow4 ? (const void*)score_kernel<DD, GG, kDbarRow4, RR, NC, ONE> \
    : dm == kDbarRow ? (const void*)score_kernel<DD, GG, kDbarRow, RR, NC, ONE>   \
    : dm == kDbarOne ? (const void*)score_kernel<DD, GG, kDbarOne, RR, NC, ONE>   \
    : dm == kDbarPair ? (const void*)score_kernel<DD, GG, kDbarPair, RR, NC, ONE> \
                      : (const void*)score_kernel<DD, GG, kDbarQuad, RR, NC, ONE>;
#define CKNV_SCORE_NC(DD, GG, RR, NC)                                             \
  if (one) { CKNV_SCORE_ONE(DD, GG, RR, NC, true) } else { CKNV_SCORE_ONE(DD, GG, RR, NC, false) }
#define CKNV_SCORE_R(DD, GG, RR)                                                  \
  if (d == DD && G == GG && a.rows == RR) {                                       \
    if (nc) { CKNV_SCORE_NC(DD, GG, RR, true) } else { CKNV_SCORE_NC(DD, GG, RR, false) } \
  }
#define CKNV_SCORE_CASE(DD) \
  CKNV_SCORE_R(DD, 1, 4) CKNV_SCORE_R(DD, 2, 4) CKNV_SCORE_R(DD, 4, 4) CKNV_SCORE_R(DD, 8, 2)
  CKNV_SCORE_CASE(64) CKNV_SCORE_CASE(128)
#undef CKNV_SCORE_CASE
#undef CKNV_SCORE_R
#undef CKNV_SCORE_NC
#undef CKNV_SCORE_ONE
  if (!f) return hipErrorInvalidValue;
  return hipLaunchKernel(f, dim3(a.nfresh + U * a.C), dim3(kScoreThreads), args, 0, st);
}

}  // namespace cknv
