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
// Grid: C workgroups ("chunks") per unit, 64 blocks each, 16 per wave; a
// block is read by 16 lanes (d/64 float4 of k̄, D̄ and v̄ each), so the wave
// reads 4 blocks' rows per load instruction. Every load is issued before
// seq_len is known; blocks past the context are masked afterwards. Per wave
// (a 16-block group) the kernel writes the LSE partial of
// a = ln|b| + z̄ + σ̂²/2 and per block u_{g,b} = exp(a - group max) σ̂²; per
// chunk it writes the Mean-compensation sums of ALL its blocks,
//   (m, l = sum |b| e^{z̄-m}, acc = sum |b| e^{z̄-m} v̄_b),
// which the attend kernel corrects by removing the kept blocks' terms (the
// kept set is not known yet). The selection kernel (select.hip) runs next.
#include "cknv_internal.h"

namespace cknv {

namespace {

// How a lane's 4 coordinates 4c..4c+3 map to D̄ entries (group size gs = d/r).
enum DbarMode { kDbarOne = 0, kDbarPair = 1, kDbarQuad = 2 };  // gs >= 4, gs == 2, gs == 1

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

template <int D, int G, int DM>
__global__ __launch_bounds__(kThreads) void score_kernel(ScoreArgs a) {
  __shared__ __align__(16) float cmb[kWaves * G * rec_words(D)];  // per-wave records
  constexpr int KC = D / 64;        // float4 chunks per lane per block (16 lanes per block)
  constexpr int ROWS = 4;           // blocks per lane: base + 4*row + (lane >> 4)
  constexpr int W = rec_words(D);

  int unit, chunk;
  map_wg(blockIdx.x, a.S * a.H, a.C, a.xcd, unit, chunk);
  const int s = unit / a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bg = lane >> 4, j = lane & 15;
  const int r = a.r, MB = a.max_blocks;
  const int base = chunk * kBlocksPerWG + wave * kBlocksPerWave;
  const size_t ubase = (size_t)unit * a.cap_blocks;

  // ---- every load of the workgroup, issued before any result is needed.
  // Block indices are clamped into [0, MB); blocks past the context are
  // masked once seq_len has arrived.
  const int T = a.seq_len[s];
  float4 qv[G][KC];
  {
    const float4* q4 = reinterpret_cast<const float4*>(a.q + (size_t)unit * G * D);
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < KC; ++i) qv[g][i] = q4[g * (D / 4) + j + 16 * i];
  }
  int blk[ROWS];
  float4 kv[ROWS][KC], vv[ROWS][KC];
  DbarTile<DM, ROWS, KC> dt;
  float n[ROWS];
  const float4* kbar4 = reinterpret_cast<const float4*>(a.kbar);
  const float4* vbar4 = reinterpret_cast<const float4*>(a.vbar);
#pragma unroll
  for (int rw = 0; rw < ROWS; ++rw) {
    blk[rw] = base + 4 * rw + bg;
    const size_t row = ubase + (blk[rw] < MB ? blk[rw] : MB - 1);
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const int c = j + 16 * i;  // float4 chunk: coordinates 4c..4c+3
      kv[rw][i] = kbar4[row * (D / 4) + c];
      vv[rw][i] = vbar4[row * (D / 4) + c];
      dt.load(a.dbar, row, c, r, D, rw, i);
    }
    n[rw] = a.cnt[row];
  }

  int NB = (T + kBlock - 1) / kBlock;
  NB = NB < MB ? NB : MB;
  bool v[ROWS];
#pragma unroll
  for (int rw = 0; rw < ROWS; ++rw) v[rw] = blk[rw] < NB;
  const bool any = base < NB;
  const float invd = 1.0f / (float)D;

  // ---- z̄ and σ̂² per (row, g): partial over the lane's coordinates, then the 16 lanes
  float z[ROWS][G], s2[ROWS][G];
#pragma unroll
  for (int rw = 0; rw < ROWS; ++rw) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float zp = 0.f, sp = 0.f;
#pragma unroll
      for (int i = 0; i < KC; ++i) {
        zp += dot4(kv[rw][i], qv[g][i]);
        sp += dt.qsq_dot(qv[g][i], rw, i);
      }
      z[rw][g] = group_sum<16>(zp) * a.isd;
      s2[rw][g] = group_sum<16>(sp) * invd;
    }
  }

  // ---- scoring partials of this wave's 16-block group
  const int gi = base / kBlocksPerWave;
  float* uo = a.u + (size_t)unit * MB * G;
  float* go = a.grp + (size_t)unit * a.NG * G * 2;
  float ln[ROWS];
#pragma unroll
  for (int rw = 0; rw < ROWS; ++rw) ln[rw] = __logf(v[rw] ? n[rw] : 1.f);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float av[ROWS], mx = -INFINITY;
#pragma unroll
    for (int rw = 0; rw < ROWS; ++rw) {
      av[rw] = v[rw] ? ln[rw] + z[rw][g] + 0.5f * s2[rw][g] : -INFINITY;
      mx = fmaxf(mx, av[rw]);
    }
    const float ref = rows_max(mx);
    float l = 0.f;
#pragma unroll
    for (int rw = 0; rw < ROWS; ++rw) {
      const float e = v[rw] ? __expf(av[rw] - ref) : 0.f;
      l += e;
      if (j == g && v[rw]) uo[(size_t)blk[rw] * G + g] = e * s2[rw][g];
    }
    l = rows_sum(l);
    if (any && lane == g) reinterpret_cast<float2*>(go)[(size_t)gi * G + g] = make_float2(ref, l);
  }

  // ---- Mean compensation of every block of the group (kept ones removed later)
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float mx = -INFINITY;
#pragma unroll
    for (int rw = 0; rw < ROWS; ++rw) mx = fmaxf(mx, v[rw] ? z[rw][g] : -INFINITY);
    const float mz = rows_max(mx);
    float w[ROWS], lz = 0.f;
#pragma unroll
    for (int rw = 0; rw < ROWS; ++rw) {
      w[rw] = v[rw] ? n[rw] * __expf(z[rw][g] - mz) : 0.f;
      lz += w[rw];
    }
    lz = rows_sum(lz);
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int rw = 0; rw < ROWS; ++rw) {
        const float wr = w[rw];
        acc.x += wr * (v[rw] ? vv[rw][i].x : 0.f);
        acc.y += wr * (v[rw] ? vv[rw][i].y : 0.f);
        acc.z += wr * (v[rw] ? vv[rw][i].z : 0.f);
        acc.w += wr * (v[rw] ? vv[rw][i].w : 0.f);
      }
      acc.x = rows_sum(acc.x);
      acc.y = rows_sum(acc.y);
      acc.z = rows_sum(acc.z);
      acc.w = rows_sum(acc.w);
      if (bg == 0) reinterpret_cast<float4*>(cmb + (wave * G + g) * W + 4)[j + 16 * i] = acc;
    }
    if (lane == 0) {
      cmb[(wave * G + g) * W] = mz;
      cmb[(wave * G + g) * W + 1] = lz;
    }
  }
  __syncthreads();
  float* co = a.comp + ((size_t)unit * a.C + chunk) * G * W;
  for (int idx = tid; idx < G * W; idx += kThreads) {
    const int g = idx / W, e = idx - g * W;
    float mw[kWaves], M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) { mw[w] = cmb[(w * G + g) * W]; M = fmaxf(M, mw[w]); }
    float val = 0.f;
    if (e == 0) {
      val = M;
    } else if (e == 1 || e >= 4) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) val += cmb[(w * G + g) * W + e] * rescale(mw[w], M);
    }
    co[idx] = val;
  }
}

hipError_t launch_score(int d, int G, const ScoreArgs& a, int U, hipStream_t st) {
  void* args[] = {(void*)&a};
  const int gs = d / a.r;
  const int dm = gs >= 4 ? kDbarOne : (gs == 2 ? kDbarPair : kDbarQuad);
  const void* f = nullptr;
#define CKNV_SCORE_CASE(DD, GG)                                         \
  if (d == DD && G == GG) {                                             \
    f = dm == kDbarOne ? (const void*)score_kernel<DD, GG, kDbarOne>    \
      : dm == kDbarPair ? (const void*)score_kernel<DD, GG, kDbarPair>  \
                        : (const void*)score_kernel<DD, GG, kDbarQuad>; \
  }
  CKNV_SCORE_CASE(64, 1) CKNV_SCORE_CASE(64, 2) CKNV_SCORE_CASE(64, 4) CKNV_SCORE_CASE(64, 8)
  CKNV_SCORE_CASE(128, 1) CKNV_SCORE_CASE(128, 2) CKNV_SCORE_CASE(128, 4) CKNV_SCORE_CASE(128, 8)
#undef CKNV_SCORE_CASE
  if (!f) return hipErrorInvalidValue;
  return hipLaunchKernel(f, dim3(U * a.C), dim3(kThreads), args, 0, st);
}

}  // namespace cknv
