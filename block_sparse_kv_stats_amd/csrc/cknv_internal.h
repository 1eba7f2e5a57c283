// Internal declarations of libcknv: workspace plan, kernel argument blocks,
// device helpers shared by the kernels. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "cknv.h"

namespace cknv {

constexpr int kBlock = 16;          // tokens per block (CompKV page, "Assumptions and limits")
constexpr int kThreads = 256;       // threads per workgroup of the score and attend kernels
constexpr int kWaves = kThreads / 64;
// Score-kernel geometry: a wave covers 4 blocks per row (16 lanes each) and
// 2 or 4 rows (a score group of 8 or 16 blocks; 2 rows at G = 8, where 4
// do not fit the registers). 4 rows halve the score groups, chunk headers
// and chunk records that every fused-step workgroup reduces afterwards
// (measured at 32K: the scoring pass takes as long with 4 rows as with 2, and
// the step kernel 0.3 us less). The selection works with either group size.
constexpr int kScoreThreads = 256;  // score kernel: 4 waves per workgroup (one chunk record each)
constexpr int kScoreWaves = kScoreThreads / 64;
constexpr int kScoreMinGroup = 8;  // blocks of the smaller score group
__host__ __device__ constexpr int score_rows(int G) { return G >= 8 ? 2 : 4; }
constexpr int kAppendThreads = 1024;
constexpr int kMaxChunksPerAttendWG = 8;  // score-chunk partials folded by one attend workgroup
constexpr int kDenseThreads = 512;        // dense attention: 8 waves per workgroup
constexpr int kDenseBlocksPerWG = 64;     // dense attention: blocks per workgroup (at least, on average)
constexpr int kDenseMaxWGs = 32;          // dense attention: workgroups per unit (at most)
constexpr int kDenseTilesInFlight = 3;   // dense attention: tiles per wave in flight (fewer than eight heads)
constexpr int kSelThreads = 512;        // selection: one workgroup per unit
constexpr int kSelKeysPerThread = 24;   // blocks per selection thread: max_blocks <= 12288

// A partial softmax record (per unit, part and query head): running max m,
// normaliser l, two pad words, then the weighted value sum acc[d]; the pad
// keeps acc 16-byte aligned.
__host__ __device__ constexpr int rec_words(int d) { return d + 4; }

// Workspace layout. All offsets in bytes from the workspace base, 256-aligned.
struct Plan {
  int U;            // units = S*H
  int NBmax;        // max_blocks
  int rows;         // score-kernel rows per wave (2 or 4)
  int bpw;          // blocks per score group = 4*rows
  int NG;           // score groups per unit (one per score wave) = ceil(NBmax/bpw)
  int Kb;           // block slots of the budget
  int C;            // score workgroups per unit = ceil(NBmax/(4*bpw))
  int P;            // attend workgroups per unit
  int Pf;           // fused-step workgroups per unit = ceil(Kb/(kStepAttendWaves*kpw))
  int pstride;      // fused-step counters per unit: 1, or 1 + ceil(Pf/8) when parts count in groups
  int kpw;          // fused step: kept blocks per attending wave
  int Pd;           // dense-attend workgroups per unit
  size_t off_grp, off_u, off_comp, off_attp, off_dense, off_t0, off_fpart, off_fphdr, off_finfo, off_hdr,
      off_pcnt, total;
};

int make_plan(const cknv_shape* sh, int max_blocks, int budget_tokens, Plan* p);

// The fused step's parts count themselves done on one counter per unit up to
// kFlatParts parts; past that, in groups of kPartGroup (one counter per
// group, whose last part then counts the group in on the unit's counter):
// same-address atomics serialise, 8 parts on one counter took 0.4 us, 32
// took 1.1 us.
constexpr int kFlatParts = 16;
constexpr int kPartGroup = 8;

struct AppendArgs {
  uint16_t* k; uint16_t* v; float* kbar; float* dbar; float* cnt; float* vbar;
  int32_t* seq_len; const uint16_t* new_k; const uint16_t* new_v;
  int S, H, r, cap_blocks;
};

struct BuildArgs {
  const uint16_t* k; const uint16_t* v; float* kbar; float* dbar; float* cnt; float* vbar;
  const int32_t* seq_len; int S, H, r, cap_blocks, max_blocks;
};

struct ScoreArgs {
  float* kbar; float* dbar; float* cnt; float* vbar;  // written only by the fresh-block workgroups
  const int32_t* seq_len; const float* q;
  float* grp; float* u; float* comp;
  float* hdr;  // per chunk and query head: (max, sum) of a over the chunk's blocks
  int S, H, r, cap_blocks, max_blocks, NG, C, xcd, rows;
  int closed_only;  // 1: score only blocks closed before this step's token (fused step)
  // Fused step only (nfresh = S*H, else 0): workgroups 0..nfresh-1 append the
  // step's token of unit blockIdx and summarise the block it lands in.
  int nfresh;
  uint16_t* k; uint16_t* v; const uint16_t* new_k; const uint16_t* new_v;
  int32_t* t0_out;  // seq_len before the step, per sequence
  float* finfo;     // per unit and query head: (a, factor of p̂ in S) of that block; a = -inf if none
  uint32_t* pcnt;   // per unit: the fused step's pstride part counters, zeroed here
  int pstride;
  int flags;        // CKNV_FLAG_* (ablation variants)
  float isd;  // 1/sqrt(d)
};

struct SelectArgs {
  const int32_t* seq_len; const float* grp; const float* u;
  const float* hdr;  // per unit, chunk and query head: (max, sum) of a over the chunk's blocks
  float* scores; int32_t* sel; int32_t* n_sel;
  int H, cap_blocks, max_blocks, NG, C, Kb, bpw_shift;
};

struct AttendArgs {
  const uint16_t* k; const uint16_t* v; const float* kbar; const float* vbar; const float* cnt;
  const int32_t* seq_len; const float* q; const int32_t* sel; const int32_t* n_sel;
  float* out; float* lse; const float* comp; float* part;
  int S, H, cap_blocks, max_blocks, Kb, C, P, xcd;
  int flags;  // CKNV_FLAG_* (ablation variants)
  float isd;
};

struct StepArgs {
  uint16_t* k; uint16_t* v; float* kbar; float* dbar; float* cnt; float* vbar;
  int32_t* seq_len; const int32_t* t0; const float* q;
  const float* grp; const float* u; const float* comp; const float* hdr;
  float* scores; int32_t* sel; int32_t* n_sel; float* out; float* lse; float* part;
  float* phdr;         // per unit, query head and part: the part record's (m, l), parts contiguous
  const float* finfo;  // per unit and query head: (a, factor) of the block the token landed in
  uint32_t* pcnt;      // per unit, pstride counters: parts done this step, then per group of
                       // kPartGroup parts (zeroed by the scoring launch)
  int pstride;
  int S, H, r, cap_blocks, max_blocks, NG, C, Kb, P, bpw_shift;
  int kpw;    // kept blocks per attending wave (a part attends kStepAttendWaves*kpw)
  int xcd;    // units a multiple of 8: a unit's parts share the XCD that scored it
  int flags;  // CKNV_FLAG_* (ablation variants)
  float isd;
};

hipError_t launch_step(int d, int G, const StepArgs& a, int U, hipStream_t st);
hipError_t launch_append(int d, const AppendArgs& a, hipStream_t st);
hipError_t launch_build(int d, const BuildArgs& a, int U, hipStream_t st);
hipError_t launch_score(int d, int G, const ScoreArgs& a, int U, hipStream_t st);
hipError_t launch_select(int G, const SelectArgs& a, int U, hipStream_t st);
hipError_t launch_attend(int d, int G, bool dense, const AttendArgs& a, int U, hipStream_t st);
hipError_t launch_zero_u32(uint32_t* p, size_t n, hipStream_t st);

// ---------------------------------------------------------------- device helpers
#ifdef __HIPCC__
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_1(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// Cross-lane data movement without the LDS: DPP within 16-lane rows, the
// gfx950 permlane swaps across rows. permlane16_swap(x, x) returns
// (rows 0,0,2,2 ; rows 1,1,3,3) and permlane32_swap(x, x) returns
// (lanes 0-31 twice ; lanes 32-63 twice), so adding the pair combines every
// lane with its xor-16 (xor-32) partner. All reductions below give every lane
// of the group the same bits (each step adds the same two operands).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16
constexpr int kDppQuadRev = 0x1B;     // quad_perm [3,2,1,0]
constexpr int kDppRor8 = 0x128;       // row_ror:8, lane i <- lane (i+8)%16 (xor 8)
constexpr int kDppBcast0 = 0x150;     // row_newbcast:k = kDppBcast0 + k, lane k of each row to the row

__device__ __forceinline__ float swap16_lo(float x, float& hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  hi = __uint_as_float(r[1]);
  return __uint_as_float(r[0]);
}
__device__ __forceinline__ float swap32_lo(float x, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  hi = __uint_as_float(r[1]);
  return __uint_as_float(r[0]);
}

// Sum / max over aligned groups of N lanes (N = 2..64), starting at lane 0 of the group.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if (N >= 2) x += dpp<kDppXor1>(x);
  if (N >= 4) x += dpp<kDppXor2>(x);
  if (N >= 8) x += dpp<kDppHalfMirror>(x);
  if (N >= 16) x += dpp<kDppMirror>(x);
  float h;
  if (N >= 32) { const float l = swap16_lo(x, h); x = l + h; }
  if (N >= 64) { const float l = swap32_lo(x, h); x = l + h; }
  return x;
}
template <int N>
__device__ __forceinline__ float group_max(float x) {
  if (N >= 2) x = fmaxf(x, dpp<kDppXor1>(x));
  if (N >= 4) x = fmaxf(x, dpp<kDppXor2>(x));
  if (N >= 8) x = fmaxf(x, dpp<kDppHalfMirror>(x));
  if (N >= 16) x = fmaxf(x, dpp<kDppMirror>(x));
  float h;
  if (N >= 32) { const float l = swap16_lo(x, h); x = fmaxf(l, h); }
  if (N >= 64) { const float l = swap32_lo(x, h); x = fmaxf(l, h); }
  return x;
}
// Sum / max over the 4 rows of the wave (lanes i, i^16, i^32, i^48).
__device__ __forceinline__ float rows_sum(float x) {
  float h;
  float l = swap16_lo(x, h);
  x = l + h;
  l = swap32_lo(x, h);
  return l + h;
}
__device__ __forceinline__ float rows_max(float x) {
  float h;
  float l = swap16_lo(x, h);
  x = fmaxf(l, h);
  l = swap32_lo(x, h);
  return fmaxf(l, h);
}

// Global loads. NT = true marks data streamed once per step (non-temporal: it
// does not displace reused lines from the caches). The hint costs latency (a
// cold random 16-token tile took 3.3 us with it against 2.8 us without, on
// MI355X), so loads on a latency-bound path use NT = false. Which streams
// gain from it was measured, not assumed: the score kernel's summary stream
// and the bulk build are faster with it (without: 130 against 119 us on the
// 16-sequence batch; 0.64 against 0.70 of peak), the dense kernel's K/V tile
// stream without it (0.53 against 0.49 of peak at 32K, 0.70 against 0.62 at
// 128K).
template <bool NT, typename V>
__device__ __forceinline__ V ldg(const V* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT = true>
__device__ __forceinline__ float4 stream_load4(const float4* p) {
  typedef float v4 __attribute__((ext_vector_type(4)));
  const v4 x = ldg<NT>(reinterpret_cast<const v4*>(p));
  return make_float4(x[0], x[1], x[2], x[3]);
}
template <bool NT = true>
__device__ __forceinline__ uint4 stream_load_u4(const uint16_t* p) {
  typedef unsigned v4 __attribute__((ext_vector_type(4)));
  const v4 x = ldg<NT>(reinterpret_cast<const v4*>(p));
  return make_uint4(x[0], x[1], x[2], x[3]);
}
template <bool NT = true>
__device__ __forceinline__ uint2 stream_load_u2(const uint16_t* p) {
  typedef unsigned v2 __attribute__((ext_vector_type(2)));
  const v2 x = ldg<NT>(reinterpret_cast<const v2*>(p));
  return make_uint2(x[0], x[1]);
}
template <bool NT = true>
__device__ __forceinline__ uint32_t stream_load_u1(const uint16_t* p) {
  return ldg<NT>(reinterpret_cast<const uint32_t*>(p));
}
template <bool NT = true>
__device__ __forceinline__ uint32_t stream_load_h(const uint16_t* p) {
  return (uint32_t)ldg<NT>(p);
}

// N consecutive floats (N = 1, 2 or a multiple of 4) from a 4N-byte aligned
// address, in vector loads of up to 16 bytes.
template <int N>
__device__ __forceinline__ void load_row(const float* p, float (&x)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const float4 v = reinterpret_cast<const float4*>(p)[i / 4];
      x[i] = v.x; x[i + 1] = v.y; x[i + 2] = v.z; x[i + 3] = v.w;
    }
  } else if constexpr (N == 2) {
    const float2 v = *reinterpret_cast<const float2*>(p);
    x[0] = v.x; x[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = p[i];
  }
}
// N float2 (the (max, sum) pairs of N query heads) from a 8N-byte aligned address.
template <int N>
__device__ __forceinline__ void load_pairs(const float2* p, float2 (&x)[N]) {
  float f[2 * N];
  load_row<2 * N>(reinterpret_cast<const float*>(p), f);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = make_float2(f[2 * i], f[2 * i + 1]);
}

// Loads of values that are the same for the whole workgroup and that no
// workgroup of the running launch writes (an earlier launch did): through
// the constant address space they become scalar loads, counted apart from
// the vector loads, so waiting for them waits for no vector load and no
// copy of a loaded vector register into a scalar one is needed.
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
typedef const __attribute__((address_space(4))) float* const_f32_ptr;
__device__ __forceinline__ int32_t load_uniform(const int32_t* p) { return *(const_i32_ptr)p; }
template <int N>
__device__ __forceinline__ void load_pairs_uniform(const float2* p, float2 (&x)[N]) {
  const_f32_ptr q = (const_f32_ptr)(const float*)p;
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = make_float2(q[2 * i], q[2 * i + 1]);
}

// Workgroup barrier for data exchanged through LDS only. __syncthreads()
// also orders global memory, so it first waits for every outstanding global
// load and store of the wave; kernels here never read in one wave what
// another wave of the workgroup wrote to global memory, so waiting for the
// wave's LDS operations is enough and in-flight global traffic keeps going.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// exp(m - M) with exp(-inf - anything) = 0 (an empty partial contributes nothing).
__device__ __forceinline__ float rescale(float m, float M) {
  return (m == -INFINITY) ? 0.f : __expf(m - M);
}

// Mean and population variance of x[0..n) (n in 1..16), x held in registers.
__device__ __forceinline__ void mean_var16(const float (&x)[16], int n, float& mean, float& var) {
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += (j < n) ? x[j] : 0.f;
  mean = s / (float)n;
  float q = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float dl = x[j] - mean;
    q += (j < n) ? dl * dl : 0.f;
  }
  var = q / (float)n;
}

// Workgroup -> (unit, part). With U a multiple of 8, all parts of a unit land
// on one XCD (workgroups are dealt to the 8 XCDs round-robin), so the
// partials a unit's last workgroup merges stay in one L2.
// (Both mappings are computed and one is selected: a branch here made the
// compiler reload the kernel argument after it, one more memory round trip
// before the first load of the workgroup.)
__device__ __forceinline__ void map_wg(int L, int U, int parts, int xcd, int& unit, int& part) {
  const int x = L & 7, y = L >> 3;
  const int yq = y / parts, lq = L / parts;
  unit = xcd ? x + 8 * yq : lq;
  part = xcd ? y - yq * parts : L - lq * parts;
}

#endif

}  // namespace cknv
