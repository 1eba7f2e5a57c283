// Attention output: exact softmax terms over the kept blocks' BF16 tokens plus
// Mean compensation of every other block, under one shared normaliser.
//
// CompKV page (onedev.kr/papers/157), "How it works" / "What differs": an
// unselected block b stands in for its |b| tokens with the block-mean logit
// z̄_b = q.k̄_b/sqrt(d) and the mean value v̄_b, contributing |b| e^{z̄_b} to
// the normaliser and |b| e^{z̄_b} v̄_b to the value sum; kept blocks use
// their tokens' exact terms, and both parts are normalised together.
//
// The score kernel already summed the compensation of ALL blocks per chunk;
// here each workgroup p of a unit
//   * adds the exact terms of its slice of the kept list (one wave per block:
//     16 tokens x d BF16 keys and values, 4 tokens per wave instruction),
//   * subtracts the kept blocks' own compensation terms |b| e^{z̄_b}(1, v̄_b),
//   * folds in its share of the score kernel's chunk sums,
// and the unit's last workgroup merges the P partials into out and lse.
// Subtracting is safe in FP32: a kept block's exact mass sum_i e^{z_i} is at
// least its compensation mass |b| e^{z̄_b} (Jensen), so the final normaliser
// is at least the sum of all compensation masses and the rounding error of
// the subtraction stays relative to the result.
//
// DENSE = true is the full-attention baseline: every block exact, no
// compensation.
#include "cknv_internal.h"

namespace cknv {

template <int D, int G, bool DENSE>
__global__ __launch_bounds__(kThreads) void attend_kernel(AttendArgs a) {
  constexpr int EPL = D / 16;  // BF16 elements per lane per token (16 lanes per token)
  constexpr int W = D + 2;
  __shared__ __align__(16) float q_l[G * D];
  __shared__ float cmb[kWaves * G * W];
  __shared__ int last;

  int unit, p;
  map_wg(blockIdx.x, a.S * a.H, a.P, a.xcd, unit, p);
  const int s = unit / a.H;
  const int T = a.seq_len[s];
  int NB = (T + kBlock - 1) / kBlock;
  NB = NB < a.max_blocks ? NB : a.max_blocks;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* qg = a.q + (size_t)unit * G * D;
  for (int i = tid; i < G * D; i += kThreads) q_l[i] = qg[i];
  __syncthreads();

  const int tq = lane >> 4, cc = lane & 15;
  const long cap_tok = (long)a.cap_blocks * kBlock;
  const size_t ubase = (size_t)unit * a.cap_blocks;

  int i0, i1;
  if (DENSE) {
    i0 = (int)((long)p * NB / a.P);
    i1 = (int)((long)(p + 1) * NB / a.P);
  } else {
    int n = a.n_sel[unit];
    n = n < a.Kb ? n : a.Kb;
    i0 = (int)((long)p * n / a.P);
    i1 = (int)((long)(p + 1) * n / a.P);
  }

  float mr[G], lr[G], acc[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    mr[g] = -INFINITY;
    lr[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
  }

  for (int it = i0 + wave; it < i1; it += kWaves) {
    const int b = DENSE ? it : a.sel[(size_t)unit * a.Kb + it];
    if (b < 0 || b >= NB) continue;  // uniform over the wave
    const long tok0 = (long)b * kBlock;
    // ---- K and V tiles: token t = 4*m + tq, lane covers coordinates [cc*EPL, +EPL)
    uint32_t kr[4][EPL / 2], vr[4][EPL / 2];
    bool tv[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int t = 4 * m + tq;
      tv[m] = tok0 + t < T;
      const size_t off = ((size_t)unit * cap_tok + tok0 + t) * D + cc * EPL;
      if (EPL == 8) {
        const uint4 z4 = make_uint4(0, 0, 0, 0);
        const uint4 kk = tv[m] ? *reinterpret_cast<const uint4*>(a.k + off) : z4;
        const uint4 vv = tv[m] ? *reinterpret_cast<const uint4*>(a.v + off) : z4;
        kr[m][0] = kk.x; kr[m][1] = kk.y; kr[m][2] = kk.z; kr[m][3] = kk.w;
        vr[m][0] = vv.x; vr[m][1] = vv.y; vr[m][2] = vv.z; vr[m][3] = vv.w;
      } else {
        const uint2 z2 = make_uint2(0, 0);
        const uint2 kk = tv[m] ? *reinterpret_cast<const uint2*>(a.k + off) : z2;
        const uint2 vv = tv[m] ? *reinterpret_cast<const uint2*>(a.v + off) : z2;
        kr[m][0] = kk.x; kr[m][1] = kk.y;
        vr[m][0] = vv.x; vr[m][1] = vv.y;
      }
    }
    float zbar[G], nb = 0.f;
    float vb[EPL];
    if (!DENSE) {
      // block-mean logit from k̄ (D/64 floats per lane, whole-wave reduce)
      constexpr int PL = D / 64;
      float kb[PL];
#pragma unroll
      for (int e = 0; e < PL; ++e) kb[e] = a.kbar[(ubase + b) * D + lane * PL + e];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float zp = 0.f;
#pragma unroll
        for (int e = 0; e < PL; ++e) zp += kb[e] * q_l[g * D + lane * PL + e];
        zbar[g] = xsum<1, 64>(zp) * a.isd;
      }
      nb = a.cnt[ubase + b];
#pragma unroll
      for (int e = 0; e < EPL; ++e) vb[e] = a.vbar[(ubase + b) * D + cc * EPL + e];
    }
    // ---- logits
    float z[4][G];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float kf[EPL];
#pragma unroll
      for (int e = 0; e < EPL / 2; ++e) { kf[2 * e] = bf16_lo(kr[m][e]); kf[2 * e + 1] = bf16_hi(kr[m][e]); }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float zp = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) zp += kf[e] * q_l[g * D + cc * EPL + e];
        zp = xsum<1, 16>(zp) * a.isd;
        z[m][g] = tv[m] ? zp : -INFINITY;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float bm = fmaxf(fmaxf(z[0][g], z[1][g]), fmaxf(z[2][g], z[3][g]));
      bm = xmax<16, 64>(bm);
      if (!DENSE) bm = fmaxf(bm, zbar[g]);
      const float M = fmaxf(mr[g], bm);
      const float sc = rescale(mr[g], M);
      lr[g] *= sc;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] *= sc;
      mr[g] = M;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float pz = tv[m] ? __expf(z[m][g] - M) : 0.f;
        lr[g] += pz;
#pragma unroll
        for (int e = 0; e < EPL / 2; ++e) {
          acc[g][2 * e] += pz * bf16_lo(vr[m][e]);
          acc[g][2 * e + 1] += pz * bf16_hi(vr[m][e]);
        }
      }
      if (!DENSE && tq == 0) {
        const float w = nb * __expf(zbar[g] - M);
        lr[g] -= w;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] -= w * vb[e];
      }
    }
  }

  // ---- sum the 4 token quarters, stage per-wave partials
#pragma unroll
  for (int g = 0; g < G; ++g) {
    lr[g] = xsum<16, 64>(lr[g]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = xsum<16, 64>(acc[g][e]);
  }
  if (tq == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < EPL; ++e) cmb[(wave * G + g) * W + 2 + cc * EPL + e] = acc[g][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      cmb[(wave * G + g) * W] = mr[g];
      cmb[(wave * G + g) * W + 1] = lr[g];
    }
  }
  __syncthreads();

  // ---- this workgroup's partial: its waves + its share of the chunk sums
  int c0 = 0, c1 = 0;
  if (!DENSE) {
    c0 = (int)((long)p * a.C / a.P);
    c1 = (int)((long)(p + 1) * a.C / a.P);
  }
  const float* comp = a.comp + (size_t)unit * a.C * G * W;
  float* po = a.part + ((size_t)unit * a.P + p) * G * W;
  for (int idx = tid; idx < G * W; idx += kThreads) {
    const int g = idx / W, e = idx - g * W;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, cmb[(w * G + g) * W]);
    for (int c = c0; c < c1; ++c) M = fmaxf(M, comp[((size_t)c * G + g) * W]);
    float val;
    if (e == 0) {
      val = M;
    } else {
      val = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) val += cmb[(w * G + g) * W + e] * rescale(cmb[(w * G + g) * W], M);
      for (int c = c0; c < c1; ++c)
        val += comp[((size_t)c * G + g) * W + e] * rescale(comp[((size_t)c * G + g) * W], M);
    }
    po[idx] = val;
  }

  if (!last_arriver(a.ctr + unit, a.P, &last)) return;
  if (tid == 0) a.ctr[unit] = 0u;
  const float* pp = a.part + (size_t)unit * a.P * G * W;
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int g = idx / D, c = idx - g * D;
    float M = -INFINITY;
    for (int q = 0; q < a.P; ++q) M = fmaxf(M, pp[((size_t)q * G + g) * W]);
    float L = 0.f, A = 0.f;
    for (int q = 0; q < a.P; ++q) {
      const float f = rescale(pp[((size_t)q * G + g) * W], M);
      L += pp[((size_t)q * G + g) * W + 1] * f;
      A += pp[((size_t)q * G + g) * W + 2 + c] * f;
    }
    const bool ok = L > 0.f;
    a.out[((size_t)unit * G + g) * D + c] = ok ? A / L : 0.f;
    if (c == 0 && a.lse) a.lse[(size_t)unit * G + g] = ok ? M + __logf(L) : -INFINITY;
  }
}

hipError_t launch_attend(int d, int G, bool dense, const AttendArgs& a, int U, hipStream_t st) {
  void* args[] = {(void*)&a};
  const void* f = nullptr;
#define CKNV_ATT_CASE(DD, GG)                                                         \
  if (d == DD && G == GG)                                                             \
    f = dense ? (const void*)attend_kernel<DD, GG, true> : (const void*)attend_kernel<DD, GG, false>;
  CKNV_ATT_CASE(64, 1) CKNV_ATT_CASE(64, 2) CKNV_ATT_CASE(64, 4) CKNV_ATT_CASE(64, 8)
  CKNV_ATT_CASE(128, 1) CKNV_ATT_CASE(128, 2) CKNV_ATT_CASE(128, 4) CKNV_ATT_CASE(128, 8)
#undef CKNV_ATT_CASE
  if (!f) return hipErrorInvalidValue;
  return hipLaunchKernel(f, dim3(U * a.P), dim3(kThreads), args, 0, st);
}

}  // namespace cknv
