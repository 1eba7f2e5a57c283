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

// Append this thread's flagged items to list[*counter ..): item m (bit m of
// `flags`) is block idx0 + m*stride with key keys[m]. One LDS atomic per
// wave reserves the wave's slots; ballots give each lane its place. Every
// lane of the wave calls this.
template <int NTILE>
__device__ __forceinline__ void list_append(uint64_t flags, const uint32_t (&keys)[NTILE], int idx0,
                                            int stride, uint64_t* list, int* counter) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (1ull << lane) - 1ull;
  uint64_t bal[NTILE];
  int tot = 0;
#pragma unroll
  for (int m = 0; m < NTILE; ++m) {
    bal[m] = __ballot((flags >> m) & 1u);
    tot += __popcll(bal[m]);
  }
  int base = 0;
  if (lane == 0 && tot > 0) base = atomicAdd(counter, tot);
  base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
  for (int m = 0; m < NTILE; ++m) {
    if ((flags >> m) & 1u) list[base + __popcll(bal[m] & below)] = rank_word(keys[m], idx0 + m * stride);
    base += __popcll(bal[m]);
  }
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

// The same exclusive prefix for callers that walk the tiles in rolled loops
// (short code: every line of a long unrolled sequence is fetched once per
// CU): returns, in lane m < NTILE of each wave, the number of flagged items
// ahead of the wave's first item of tile m (read per tile with readlane);
// the total goes to *total. `cnt`: LDS scratch of NTILE*NW + 1 ints. Every
// thread calls this.
template <int NTILE, int NW>
__device__ __forceinline__ int tile_bases(uint64_t flags, int* cnt, int& total) {
  static_assert(NTILE <= 64, "one lane per tile");
  constexpr int E = NTILE * NW;
  constexpr int PER = (E + 63) / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int mine = 0;
#pragma unroll 1
  for (int m = 0; m < NTILE; ++m) {
    const int c = __popcll(__ballot((flags >> m) & 1u));
    mine = lane == m ? c : mine;
  }
  if (lane < NTILE) cnt[lane * NW + wave] = mine;
  lds_barrier();
  if (wave == 0) {
    int v[PER], own = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = lane * PER + k;
      v[k] = i < E ? cnt[i] : 0;
      own += v[k];
    }
    const int incl = wave_incl_scan(own);
    int run = incl - own;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = lane * PER + k;
      if (i < E) cnt[i] = run;
      run += v[k];
    }
    if (lane == 63) cnt[E] = incl;
  }
  lds_barrier();
  total = cnt[E];
  return lane < NTILE ? cnt[lane * NW + wave] : 0;
}

// Exclusive prefix over items in tile-major order: tile m holds items
// m*NT .. m*NT+NT-1 (thread t's item of tile m is m*NT + t); bit m of
// `flags` is this thread's flag in tile m. before[m] gets the number of
// flagged items ahead of this thread's item of tile m; the total goes to
// *total. `cnt`: LDS scratch of NTILE*NW + 1 ints. Every thread calls this.
template <int NTILE, int NW>
__device__ __forceinline__ void tile_prefix(uint64_t flags, int (&before)[NTILE], int* cnt,
                                            int& total) {
  constexpr int E = NTILE * NW;       // (tile, wave) entries in item order
  constexpr int PER = (E + 63) / 64;  // entries per lane of wave 0
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int m = 0; m < NTILE; ++m) {
    const unsigned long long bal = __ballot((flags >> m) & 1u);
    before[m] = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) cnt[m * NW + wave] = __popcll(bal);
  }
  lds_barrier();
  if (wave == 0) {  // exclusive scan of the E counts, in place; total after them
    int v[PER], own = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = lane * PER + k;
      v[k] = i < E ? cnt[i] : 0;
      own += v[k];
    }
    const int incl = wave_incl_scan(own);
    int run = incl - own;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = lane * PER + k;
      if (i < E) cnt[i] = run;
      run += v[k];
    }
    if (lane == 63) cnt[E] = incl;
  }
  lds_barrier();
#pragma unroll
  for (int m = 0; m < NTILE; ++m) before[m] += cnt[m * NW + wave];
  total = cnt[E];
}

}  // namespace cknv
