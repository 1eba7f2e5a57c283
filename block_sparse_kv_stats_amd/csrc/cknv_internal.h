// Internal declarations of libcknv: workspace plan, kernel argument blocks,
// device helpers shared by the kernels. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "cknv.h"

namespace cknv {

constexpr int kBlock = 16;          // tokens per block (CompKV page, "Assumptions and limits")
constexpr int kThreads = 256;       // threads per workgroup of every streaming kernel
constexpr int kWaves = kThreads / 64;
constexpr int kBlocksPerWave = 16;  // one 16-block score group per wave iteration
constexpr int kBlocksPerIter = kWaves * kBlocksPerWave;
constexpr int kMaxChunks = 64;      // score workgroups per unit, at most
constexpr int kDenseTargetWGs = 1024;
constexpr size_t kMaxLds = 64 * 1024;

// Workspace layout. All offsets in bytes from the workspace base, 256-aligned.
struct Plan {
  int U;            // units = S*H
  int NBmax;        // max_blocks
  int NG;           // 16-block score groups per unit = ceil(NBmax/16)
  int Kb;           // block slots of the budget
  int C;            // score chunks (workgroups) per unit
  int BPC;          // blocks per score chunk (multiple of 64)
  int P;            // attend workgroups per unit
  int Pd;           // dense-attend workgroups per unit
  size_t off_ctr, off_grp, off_u, off_comp, off_attp, off_dense, total;
  size_t n_ctr;     // counters (uint32)
  size_t score_lds; // dynamic LDS of the score kernel
};

// Counter rows inside the counter region (uint32 each, row length = max(S, U)).
enum { kCtrAppend = 0, kCtrScore = 1, kCtrAttend = 2, kCtrDense = 3, kCtrRows = 4 };

int make_plan(const cknv_shape* sh, int max_blocks, int budget_tokens, Plan* p);

struct AppendArgs {
  uint16_t* k; uint16_t* v; float* kbar; float* dbar; float* cnt; float* vbar;
  int32_t* seq_len; const uint16_t* new_k; const uint16_t* new_v; uint32_t* ctr;
  int S, H, r, cap_blocks;
};

struct BuildArgs {
  const uint16_t* k; const uint16_t* v; float* kbar; float* dbar; float* cnt; float* vbar;
  const int32_t* seq_len; int S, H, r, cap_blocks, max_blocks;
};

struct ScoreArgs {
  const float* kbar; const float* dbar; const float* cnt; const float* vbar;
  const int32_t* seq_len; const float* q;
  float* scores; int32_t* sel; int32_t* n_sel;
  uint32_t* ctr; float* grp; float* u; float* comp;
  int S, H, r, cap_blocks, max_blocks, NG, Kb, C, BPC, xcd;
  float isd;  // 1/sqrt(d)
};

struct AttendArgs {
  const uint16_t* k; const uint16_t* v; const float* kbar; const float* vbar; const float* cnt;
  const int32_t* seq_len; const float* q; const int32_t* sel; const int32_t* n_sel;
  float* out; float* lse; uint32_t* ctr; const float* comp; float* part;
  int S, H, cap_blocks, max_blocks, Kb, C, P, xcd;
  float isd;
};

hipError_t launch_append(int d, const AppendArgs& a, int U, hipStream_t st);
hipError_t launch_build(int d, const BuildArgs& a, int U, hipStream_t st);
hipError_t launch_score(int d, int G, const ScoreArgs& a, int U, size_t lds, hipStream_t st);
hipError_t launch_attend(int d, int G, bool dense, const AttendArgs& a, int U, hipStream_t st);
hipError_t launch_zero_u32(uint32_t* p, size_t n, hipStream_t st);

// ---------------------------------------------------------------- device helpers
#ifdef __HIPCC__
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_1(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// Sum / max over the lanes whose index differs from this lane's in the bits
// LO, 2*LO, ..., below HI (butterfly, every participating lane gets the result).
template <int LO, int HI>
__device__ __forceinline__ float xsum(float x) {
#pragma unroll
  for (int o = LO; o < HI; o <<= 1) x += __shfl_xor(x, o);
  return x;
}
template <int LO, int HI>
__device__ __forceinline__ float xmax(float x) {
#pragma unroll
  for (int o = LO; o < HI; o <<= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// exp(m - M) with exp(-inf - anything) = 0 (an empty partial contributes nothing).
__device__ __forceinline__ float rescale(float m, float M) {
  return (m == -INFINITY) ? 0.f : __expf(m - M);
}

// Workgroup -> (unit, part). With U a multiple of 8, all parts of a unit land
// on one XCD (workgroups are dealt to the 8 XCDs round-robin), so the
// partials a unit's last workgroup merges stay in one L2.
__device__ __forceinline__ void map_wg(int L, int U, int parts, int xcd, int& unit, int& part) {
  if (xcd) {
    const int x = L & 7, y = L >> 3;
    unit = x + 8 * (y / parts);
    part = y % parts;
  } else {
    unit = L / parts;
    part = L % parts;
  }
}

// Last-arriver election among the `expected` workgroups of one unit. Every
// thread fences its own global writes (release) before the barrier; the
// returned flag is uniform over the workgroup. The winner fences again
// (acquire) before reading what the others wrote.
__device__ __forceinline__ bool last_arriver(uint32_t* ctr, int expected, int* flag_lds) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = atomicAdd(ctr, 1u);
    *flag_lds = (prev == (uint32_t)(expected - 1));
  }
  __syncthreads();
  const bool last = *flag_lds != 0;
  if (last) __threadfence();
  return last;
}
#endif

}  // namespace cknv
