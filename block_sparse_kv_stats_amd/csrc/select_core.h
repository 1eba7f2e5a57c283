// Device helpers of the block selection shared by the selection kernels.
// Internal to libcknv.
#pragma once

#include "cknv_internal.h"

namespace cknv {

constexpr int kListMax = 256;  // pivot-bin keys ranked exactly; more go to the radix fallback

// Inclusive prefix sum over the 64 lanes of a wave without the LDS: a
// log-step scan inside each 16-lane row (DPP row_shr 1, 2, 4, 8; lanes
// shifted in from outside the row read 0), then each row adds the totals of
// the rows before it (read from lanes 15, 31, 47).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_mov_dpp(x, 0x111, 0xF, 0xF, true);
  x += __builtin_amdgcn_mov_dpp(x, 0x112, 0xF, 0xF, true);
  x += __builtin_amdgcn_mov_dpp(x, 0x114, 0xF, 0xF, true);
  x += __builtin_amdgcn_mov_dpp(x, 0x118, 0xF, 0xF, true);
  const int t0 = __builtin_amdgcn_readlane(x, 15), t1 = __builtin_amdgcn_readlane(x, 31);
  const int t2 = __builtin_amdgcn_readlane(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row >= 1 ? t0 : 0) + (row >= 2 ? t1 : 0) + (row >= 3 ? t2 : 0);
}

// Wave 0: the bin of `hist` (NBINS bins, higher bin = larger keys) holding
// the krem-th largest counted key; writes (bin, rank within the bin, count
// in the bin) to ctl[0..2]. Lane l owns bins [l*PER, (l+1)*PER).
template <int NBINS>
__device__ __forceinline__ void find_bin(const int* hist, int krem, int* ctl) {
  constexpr int PER = NBINS / 64, NC = PER / 4;
  const int lane = threadIdx.x & 63;
  const int4* h4 = reinterpret_cast<const int4*>(hist + lane * PER);
  int cs[NC], own = 0;  // per int4 chunk of bins
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int4 v = h4[i];
    cs[i] = v.x + v.y + v.z + v.w;
    own += cs[i];
  }
  const int incl = wave_incl_scan(own);
  const int total = __builtin_amdgcn_readlane(incl, 63);
  int cum = total - incl;  // keys in bins of higher lanes
  if (cum < krem && krem <= cum + own) {  // this lane holds the bin
    int ci = 0, cb = cum;                  // chunk holding it, keys above that chunk
    int c = cum;
#pragma unroll
    for (int i = NC - 1; i >= 0; --i) {
      if (c < krem && krem <= c + cs[i]) { ci = i; cb = c; }
      c += cs[i];
    }
    const int4 v = h4[ci];
    const int hv[4] = {v.x, v.y, v.z, v.w};
    c = cb;
#pragma unroll
    for (int e = 3; e >= 0; --e) {
      if (c < krem && krem <= c + hv[e]) {
        ctl[0] = lane * PER + 4 * ci + e;
        ctl[1] = krem - c;
        ctl[2] = hv[e];
      }
      c += hv[e];
    }
  }
}

// A pivot-bin key and its block index as one word that orders like the
// selection, (key desc, index asc): the key in the high half, the index's
// complement in the low half. Every such word is nonzero, so zero words can
// pad a list without ranking above any entry.
__device__ __forceinline__ uint64_t rank_word(uint32_t key, int idx) {
  return ((uint64_t)key << 32) | (uint64_t)(0xffffffffu - (uint32_t)idx);
}

// Ranks of the n words of `list` (followed by at least kListPad zero words):
// an entry is kept when fewer than krem entries order above it; its block's
// bit is set in keep_bits. Thread t ranks entries t, t+NT, ...; 32 words are
// read per LDS round trip.
constexpr int kListPad = 32;
template <int NT>
__device__ __forceinline__ void rank_list_keep(const uint64_t* list, int n, int krem, uint32_t* keep_bits) {
  for (int i = threadIdx.x; i < n; i += NT) {
    const uint64_t ci = list[i];
    int rank = 0;
    for (int j0 = 0; j0 < n; j0 += kListPad) {
      ulonglong2 v[kListPad / 2];
#pragma unroll
      for (int e = 0; e < kListPad / 2; ++e) v[e] = reinterpret_cast<const ulonglong2*>(list + j0)[e];
#pragma unroll
      for (int e = 0; e < kListPad / 2; ++e) rank += (int)(v[e].x > ci) + (int)(v[e].y > ci);
    }
    if (rank < krem) {
      const int ii = (int)(0xffffffffu - (uint32_t)ci);
      atomicOr(&keep_bits[ii >> 5], 1u << (ii & 31));
    }
  }
}

// Append the flagged entries of this thread's run of blocks b0, b0+1, ...
// (bit i of `flags`: block b0 + i, whose key is keys[b0 + i], keys in LDS)
// to list[*counter ..): one LDS atomic per wave reserves the wave's entries,
// a wave scan of the per-thread counts places each thread's, and a thread
// visits only its flagged blocks. Every lane of the wave calls this.
__device__ __forceinline__ void run_append(uint64_t flags, const uint32_t* keys, int b0,
                                           uint64_t* list, int* counter) {
  const int lane = threadIdx.x & 63;
  const int n = __popcll(flags);
  const int incl = wave_incl_scan(n);
  const int tot = __builtin_amdgcn_readlane(incl, 63);
  int base = 0;
  if (lane == 0 && tot > 0) base = atomicAdd(counter, tot);
  base = __builtin_amdgcn_readfirstlane(base) + incl - n;
  for (uint64_t m = flags; m; m &= m - 1) {
    const int b = b0 + (int)__builtin_ctzll(m);
    list[base++] = rank_word(keys[b], b);
  }
}

// Exclusive prefix sum of x over the workgroup's threads in thread order;
// the sum of all goes to *total. `tmp`: LDS scratch of NW ints, free on entry
// (the caller puts a barrier between two calls). Every thread calls this.
template <int NW>
__device__ __forceinline__ int block_excl_scan(int x, int* tmp, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(x);
  if (lane == 63) tmp[wave] = incl;
  lds_barrier();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int c = tmp[w];
    before += w < wave ? c : 0;
    tot += c;
  }
  total = tot;
  return before + incl - x;
}

}  // namespace cknv
