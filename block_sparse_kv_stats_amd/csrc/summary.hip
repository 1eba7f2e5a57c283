// Block-summary kernels: the per-step append (new token + open-block
// refresh) and the bulk build of every block's summary from the cache.
//
// CompKV page (onedev.kr/papers/157), "What differs": a block's summary is
// {|b|, mean key, D̄_b, mean value}, where D̄_b holds for each of the r groups
// of key coordinates the mean of those coordinates' variances.
// "How to use it": every decode step a fused kernel refreshes the current
// block's statistics and stores the new K/V.
//
// Both recompute a block from its (at most 16) BF16 tokens: two passes in
// FP32 (mean, then the mean squared deviation, i.e. the population
// variance), summed in token order; D̄ groups summed as a balanced pairwise
// tree. The bulk build and the fused step's refresh share summary_core.h.
#include "cknv_internal.h"
#include "summary_core.h"

namespace cknv {

// D̄_t = mean of the coordinate variances of group t = [t*gs, (t+1)*gs).
// The D coordinate variances of `nslot` blocks sit in cvar[slot*D + c]; the
// workgroup sums each group as a balanced pairwise tree (each node = left +
// right, the order a lane butterfly gives), leaving the sum in cvar[t*gs].
// Every thread of the workgroup must call this.
template <int D, int NTH>
__device__ __forceinline__ void group_tree_sums(float* cvar, int nslot, int gs) {
  for (int len = 1; len < gs; len <<= 1) {
    lds_barrier();
    for (int i = threadIdx.x; i < nslot * D; i += NTH) {
      const int c = i % D;
      if (c % (2 * len) == 0) cvar[i] += cvar[i + len];
    }
  }
  lds_barrier();
}

// One workgroup per sequence: thread (h, c) handles key coordinate c of head
// h (looping when H*D exceeds the workgroup). The token is written and the
// block refreshed for every head before seq_len[s] advances, so no other
// workgroup reads seq_len[s] concurrently.
template <int D>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
  __shared__ float cvar[kAppendThreads];
  constexpr int HPI = kAppendThreads / D;  // heads per pass
  const int s = blockIdx.x;
  const int T = a.seq_len[s];
  const long cap_tok = (long)a.cap_blocks * kBlock;
  const bool room = T < cap_tok;
  const int b = T / kBlock;
  const int n = T - b * kBlock + 1;  // tokens in the block once the new one is in
  const int hl = threadIdx.x / D, c = threadIdx.x % D;
  const int gs = D / a.r;
  for (int h0 = 0; h0 < a.H; h0 += HPI) {
    const int h = h0 + hl;
    const bool act = room && h < a.H;
    const int unit = s * a.H + h;
    const size_t row = (size_t)unit * a.cap_blocks + b;
    float kv = 0.f;
    if (act) {
      const size_t tok0 = (size_t)unit * cap_tok + (size_t)b * kBlock;
      const uint16_t* kb = a.k + tok0 * D + c;
      const uint16_t* vb = a.v + tok0 * D + c;
      const uint16_t nk = a.new_k[(size_t)unit * D + c];
      const uint16_t nv = a.new_v[(size_t)unit * D + c];
      // all 16 rows are read (the block lies inside the cache); rows at or
      // past the new token's are replaced or masked at use, so every load is
      // issued before the first one is used
      uint16_t kr[16], vr[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        kr[j] = kb[(size_t)j * D];
        vr[j] = vb[(size_t)j * D];
      }
      float kx[16], vx[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const bool old = j < n - 1;
        kx[j] = j < n ? bf16_1(old ? kr[j] : nk) : 0.f;
        vx[j] = j < n ? bf16_1(old ? vr[j] : nv) : 0.f;
      }
      a.k[(tok0 + n - 1) * D + c] = nk;
      a.v[(tok0 + n - 1) * D + c] = nv;
      float km, vm, vv;
      mean_var16(kx, n, km, kv);
      mean_var16(vx, n, vm, vv);
      a.kbar[row * D + c] = km;
      a.vbar[row * D + c] = vm;
      if (c == 0) a.cnt[row] = (float)n;
    }
    if (gs <= 64) {
      // a group lies within the wave (coordinates c of one head are lanes):
      // the same balanced pairwise tree by lane exchanges (lane c adds lane
      // c^len: left + right, or right + left, which is the same sum)
      float x = kv;
      for (int len = 1; len < gs; len <<= 1) x += __shfl_xor(x, len);
      if (act && c % gs == 0) a.dbar[row * a.r + c / gs] = x / (float)gs;
    } else {
      lds_barrier();
      cvar[threadIdx.x] = kv;
      group_tree_sums<D, kAppendThreads>(cvar, HPI, gs);
      if (act && c % gs == 0) a.dbar[row * a.r + c / gs] = cvar[threadIdx.x] / (float)gs;
      lds_barrier();
    }
  }
  if (threadIdx.x == 0 && room) a.seq_len[s] = T + 1;
}

// Bulk build: one wave per block (kWaves blocks per workgroup), lane l owning
// coordinates [l*VPL, l*VPL + VPL) of all its tokens; every load of the wave
// is issued before the first use. Blocks at or past NB are left untouched.
template <int D>
__global__ __launch_bounds__(kThreads) void build_kernel(BuildArgs a) {
  constexpr int VPL = D / 64;
  const int unit = blockIdx.y, s = unit / a.H;
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int T = a.seq_len[s];
  int NB = (T + kBlock - 1) / kBlock;
  NB = NB < a.max_blocks ? NB : a.max_blocks;
  if (b >= NB) return;  // wave-uniform
  const int n = (T - b * kBlock) < kBlock ? (T - b * kBlock) : kBlock;
  const long cap_tok = (long)a.cap_blocks * kBlock;
  const uint16_t* kc = a.k + (size_t)unit * cap_tok * D;
  const uint16_t* vc = a.v + (size_t)unit * cap_tok * D;
  uint32_t fk[16], fv[16];
  load_block_words<D, true>(kc, vc, (long)b * kBlock, n, lane, fk, fv);
  float km[VPL], vm[VPL], dl[VPL];
  block_summary<D>(fk, fv, n, a.r, km, vm, dl);
  store_block_summary<D>(a.kbar, a.dbar, a.cnt, a.vbar, (size_t)unit * a.cap_blocks + b, a.r, n,
                         lane, km, vm, dl);
}

__global__ void zero_u32_kernel(uint32_t* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

hipError_t launch_append(int d, const AppendArgs& a, hipStream_t st) {
  void* args[] = {(void*)&a};
  const void* f = d == 128 ? (const void*)append_kernel<128> : (const void*)append_kernel<64>;
  return hipLaunchKernel(f, dim3(a.S), dim3(kAppendThreads), args, 0, st);
}

hipError_t launch_build(int d, const BuildArgs& a, int U, hipStream_t st) {
  void* args[] = {(void*)&a};
  const int gx = (a.max_blocks + kWaves - 1) / kWaves;
  const void* f = d == 128 ? (const void*)build_kernel<128> : (const void*)build_kernel<64>;
  return hipLaunchKernel(f, dim3(gx, U), dim3(kThreads), args, 0, st);
}

hipError_t launch_zero_u32(uint32_t* p, size_t n, hipStream_t st) {
  void* args[] = {(void*)&p, (void*)&n};
  const unsigned g = (unsigned)((n + 255) / 256);
  return hipLaunchKernel((const void*)zero_u32_kernel, dim3(g ? g : 1), dim3(256), args, 0, st);
}

}  // namespace cknv
