// The summary of one 16-token block, computed by one wave: lane l owns key
// and value coordinates [l*VPL, l*VPL + VPL) (VPL = d/64) of every token.
// Shared by the bulk build and the fused step's refresh of the block a new
// token lands in, so a summary kept up to date step by step equals one
// rebuilt from the cache bit for bit. Internal to libcknv.
//
// CompKV page (onedev.kr/papers/157), "What differs": a block's summary is
// {|b|, mean key, D̄, mean value}, D̄ holding for each of the r contiguous
// groups of key coordinates the mean of those coordinates' (population)
// variances.
#pragma once

#include "cknv_internal.h"

namespace cknv {

// The lane's words of n (1..16) tokens: token j of the block from the cache
// row at tok (slots past the last valid one read the last valid token; they
// are not used). d = 128: one word holds the lane's 2 bf16, d = 64: the low
// half holds its 1 bf16. NT: non-temporal loads (a bulk pass) or plain ones.
template <int D, bool NT>
__device__ __forceinline__ void load_block_words(const uint16_t* kc, const uint16_t* vc, long tok0,
                                                 int n, int lane, uint32_t (&fk)[16],
                                                 uint32_t (&fv)[16]) {
  constexpr int VPL = D / 64;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const long t = tok0 + (j < n ? j : (n > 0 ? n - 1 : 0));
    const size_t off = (size_t)t * D + lane * VPL;
    fk[j] = VPL == 2 ? stream_load_u1<NT>(kc + off) : stream_load_h<NT>(kc + off);
    fv[j] = VPL == 2 ? stream_load_u1<NT>(vc + off) : stream_load_h<NT>(vc + off);
  }
}

// Summary of the n tokens in fk/fv: the lane's coordinates of k̄ and v̄, and
// dl[e] = D̄ of the group holding coordinate l*VPL + e (the same in every
// lane of the group). Mean and variance are two passes over the tokens in
// order; each group's variances are summed as a balanced pairwise tree
// (in-lane pair, then lane butterflies: every step adds the same two values
// in both lanes). Every lane of the wave must call it.
template <int D>
__device__ __forceinline__ void block_summary(const uint32_t (&fk)[16], const uint32_t (&fv)[16],
                                              int n, int r, float (&km)[D / 64],
                                              float (&vm)[D / 64], float (&dl)[D / 64]) {
  constexpr int VPL = D / 64;
  float kvr[VPL];
#pragma unroll
  for (int e = 0; e < VPL; ++e) {
    float kx[16], vx[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      kx[j] = e == 0 ? bf16_lo(fk[j]) : bf16_hi(fk[j]);
      vx[j] = e == 0 ? bf16_lo(fv[j]) : bf16_hi(fv[j]);
    }
    float vvar;
    mean_var16(kx, n, km[e], kvr[e]);
    mean_var16(vx, n, vm[e], vvar);
  }
  const int gs = D / r;
  if (gs >= VPL) {
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < VPL; ++e) part += kvr[e];
    switch (gs / VPL) {  // lanes per group: a butterfly sum (DPP and row swaps)
      case 2: part = group_sum<2>(part); break;
      case 4: part = group_sum<4>(part); break;
      case 8: part = group_sum<8>(part); break;
      case 16: part = group_sum<16>(part); break;
      case 32: part = group_sum<32>(part); break;
      case 64: part = group_sum<64>(part); break;
      default: break;
    }
#pragma unroll
    for (int e = 0; e < VPL; ++e) dl[e] = part / (float)gs;
  } else {
#pragma unroll
    for (int e = 0; e < VPL; ++e) dl[e] = kvr[e];
  }
}

// Store a block summary (row = unit*cap_blocks + block) from block_summary.
template <int D>
__device__ __forceinline__ void store_block_summary(float* kbar, float* dbar, float* cnt, float* vbar,
                                                    size_t row, int r, int n, int lane,
                                                    const float (&km)[D / 64], const float (&vm)[D / 64],
                                                    const float (&dl)[D / 64]) {
  constexpr int VPL = D / 64;
  const int gs = D / r;
#pragma unroll
  for (int e = 0; e < VPL; ++e) {
    kbar[row * D + lane * VPL + e] = km[e];
    vbar[row * D + lane * VPL + e] = vm[e];
  }
  if (gs >= VPL) {
    if ((lane * VPL) % gs == 0) dbar[row * r + (lane * VPL) / gs] = dl[0];
  } else {
#pragma unroll
    for (int e = 0; e < VPL; ++e) dbar[row * r + lane * VPL + e] = dl[e];
  }
  if (lane == 0) cnt[row] = (float)n;
}

}  // namespace cknv
