// Block scoring and selection, one streaming pass over the summary store.
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
//
// Grid: C workgroups ("chunks") per unit, each streaming BPC blocks of k̄,
// D̄, |b| and v̄. Per 16-block group a wave writes the LSE partial of
// a = ln|b| + z̄ + σ̂²/2 and per block u_{g,b} = exp(a - group max) σ̂²; per
// chunk the workgroup writes the Mean-compensation sums of ALL its blocks,
//   (m, l = sum |b| e^{z̄-m}, acc = sum |b| e^{z̄-m} v̄_b),
// which the attend kernel later corrects by removing the kept blocks' terms
// (the kept set is not known yet). The last chunk of a unit to finish
// normalises the scores (S_b = sum_g u_{g,b} e^{max - LSE_g}) and runs an
// MSB-first radix select on the fp32 bit patterns of S_b (S_b >= 0, so the
// bit patterns order like the values) with ties to the lower index.
#include "cknv_internal.h"

namespace cknv {

namespace {

__device__ __forceinline__ float dot4(const float4 a, const float4 b) {
  return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}

// Wave-level LDS hand-off: orders this wave's LDS writes before its reads.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Exclusive prefix sum of one int per thread over the 256-thread workgroup.
__device__ int block_exclusive_scan(int v, int* scratch /*>= 5 ints*/, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int t = scratch[w];
    before += (w < wave) ? t : 0;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return before + x - v;
}

__device__ __forceinline__ int kpad(int b) { return b + (b >> 5); }

// The selection, run by the unit's last workgroup. LDS use (bytes):
// keys kpad(NBmax)+1 words, f NG*G floats, small scratch.
template <int G>
__device__ void select_tail(const ScoreArgs& a, int unit, int NB, unsigned char* lds) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t* keys = reinterpret_cast<uint32_t*>(lds);
  float* f = reinterpret_cast<float*>(keys + kpad(a.max_blocks) + 1);
  float* red = f + (size_t)a.NG * G;                 // [kWaves][G][2] + [G]
  int* hist = reinterpret_cast<int*>(red + kWaves * G * 2 + G + 3);  // [256]
  int* scr = hist + 256;                              // scan scratch + digit hand-off
  int32_t* sel = a.sel + (size_t)unit * a.Kb;

  if (tid == 0) a.ctr[unit] = 0u;
  if (NB == 0) {
    if (tid == 0) a.n_sel[unit] = 0;
    return;
  }
  const int NGu = (NB + kBlocksPerWave - 1) / kBlocksPerWave;
  const float* grp = a.grp + (size_t)unit * a.NG * G * 2;

  // LSE_g over all blocks from the per-group (max, sum) partials.
  float m[G], sm[G];
#pragma unroll
  for (int g = 0; g < G; ++g) { m[g] = -INFINITY; sm[g] = 0.f; }
  for (int gi = tid; gi < NGu; gi += kThreads) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float r = grp[(gi * G + g) * 2], l = grp[(gi * G + g) * 2 + 1];
      const float M = fmaxf(m[g], r);
      sm[g] = sm[g] * rescale(m[g], M) + l * rescale(r, M);
      m[g] = M;
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float m2 = __shfl_xor(m[g], o), s2 = __shfl_xor(sm[g], o);
      const float M = fmaxf(m[g], m2);
      sm[g] = sm[g] * rescale(m[g], M) + s2 * rescale(m2, M);
      m[g] = M;
    }
    if (lane == 0) { red[(wave * G + g) * 2] = m[g]; red[(wave * G + g) * 2 + 1] = sm[g]; }
  }
  __syncthreads();
  float* lse = red + kWaves * G * 2;
  if (tid < G) {
    float M = -INFINITY, L = 0.f;
    for (int w = 0; w < kWaves; ++w) {
      const float m2 = red[(w * G + tid) * 2], s2 = red[(w * G + tid) * 2 + 1];
      const float MM = fmaxf(M, m2);
      L = L * rescale(M, MM) + s2 * rescale(m2, MM);
      M = MM;
    }
    lse[tid] = M + __logf(L);
  }
  __syncthreads();
  for (int i = tid; i < NGu * G; i += kThreads) f[i] = __expf(grp[i * 2] - lse[i % G]);
  __syncthreads();

  // S_b and its key.
  const float* u = a.u + (size_t)unit * a.max_blocks * G;
  float* scores = a.scores ? a.scores + (size_t)unit * a.cap_blocks : nullptr;
  for (int b = tid; b < NB; b += kThreads) {
    float S = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) S += u[(size_t)b * G + g] * f[(b >> 4) * G + g];
    keys[kpad(b)] = S > 0.f ? __float_as_uint(S) : 0u;
    if (scores) scores[b] = S;
  }
  __syncthreads();

  if (NB <= a.Kb) {
    for (int b = tid; b < NB; b += kThreads) sel[b] = b;
    if (tid == 0) a.n_sel[unit] = NB;
    return;
  }

  // Radix select of the (Kb-3)-th largest key among candidates 1..NB-3.
  // With Kb = 3 only the forced set is kept: the threshold is above every key.
  uint32_t prefix = 0u;
  int krem = a.Kb - 3;
  const int passes = krem > 0 ? 4 : 0;
  if (krem == 0) prefix = 0xffffffffu;
#pragma unroll 1
  for (int pass = 0; pass < passes; ++pass) {
    const int shift = 24 - 8 * pass;
    const uint32_t hmask = pass == 0 ? 0u : (0xffffffffu << (shift + 8));
    hist[tid] = 0;
    __syncthreads();
    for (int b = 1 + tid; b <= NB - 3; b += kThreads) {
      const uint32_t key = keys[kpad(b)];
      if ((key & hmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
    }
    __syncthreads();
    if (wave == 0) {
      // lane owns bins 4*lane .. 4*lane+3; count of keys in higher bins
      int h[4], own = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) { h[e] = hist[4 * lane + e]; own += h[e]; }
      int above = own;  // inclusive suffix over lanes >= lane
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_down(above, o);
        if (lane + o < 64) above += y;
      }
      int cum = above - own;  // keys in bins of higher lanes
#pragma unroll
      for (int e = 3; e >= 0; --e) {
        if (cum < krem && krem <= cum + h[e]) {
          scr[8] = 4 * lane + e;
          scr[9] = krem - cum;
        }
        cum += h[e];
      }
    }
    __syncthreads();
    prefix |= ((uint32_t)scr[8]) << shift;
    krem = scr[9];
    __syncthreads();
  }
  const uint32_t tau = prefix;

  // Ascending compaction: thread t owns blocks [t*per, (t+1)*per).
  const int per = (NB + kThreads - 1) / kThreads;
  const int lo = tid * per, hi = min(NB, lo + per);
  int n_eq = 0, n_take = 0;
  for (int b = lo; b < hi; ++b) {
    const bool forced = (b == 0) || (b >= NB - 2);
    const uint32_t key = keys[kpad(b)];
    n_eq += (!forced && key == tau);
    n_take += forced || key > tau;
  }
  int tot;
  const int eq_before = block_exclusive_scan(n_eq, scr, tot);
  int my_eq = krem - eq_before;
  my_eq = my_eq < 0 ? 0 : (my_eq > n_eq ? n_eq : my_eq);
  int pos = block_exclusive_scan(n_take + my_eq, scr, tot);
  for (int b = lo; b < hi; ++b) {
    const bool forced = (b == 0) || (b >= NB - 2);
    const uint32_t key = keys[kpad(b)];
    bool take = forced || key > tau;
    if (!forced && key == tau && my_eq > 0) { take = true; --my_eq; }
    if (take) sel[pos++] = b;
  }
  if (tid == 0) a.n_sel[unit] = a.Kb;
}

}  // namespace

template <int D, int G>
__global__ __launch_bounds__(kThreads) void score_kernel(ScoreArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  __shared__ int last;
  constexpr int KC = D / 32;        // float4 of k̄ per lane per block (8 lanes per block)
  constexpr int LPBV = D / 4;       // lanes per block when streaming v̄ as float4
  constexpr int BPIV = 64 / LPBV;   // blocks per v̄ load instruction
  constexpr int NV = kBlocksPerWave / BPIV;
  constexpr int W = D + 2;

  int unit, chunk;
  map_wg(blockIdx.x, a.S * a.H, a.C, a.xcd, unit, chunk);
  const int s = unit / a.H;
  const int T = a.seq_len[s];
  int NB = (T + kBlock - 1) / kBlock;
  NB = NB < a.max_blocks ? NB : a.max_blocks;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = a.r;
  float* q_l = reinterpret_cast<float*>(lds);   // [G][D]
  float* qe_l = q_l + G * D;                    // [G][r]
  float* w_l = qe_l + G * r;                    // [kWaves][16][G]
  float* cmb = w_l + kWaves * 16 * G;           // [kWaves][G][W]

  const float* qg = a.q + (size_t)unit * G * D;
  for (int i = tid; i < G * D; i += kThreads) q_l[i] = qg[i];
  __syncthreads();
  const int gs = D / r;
  for (int i = tid; i < G * r; i += kThreads) {
    const int g = i / r, t = i - g * r;
    float e = 0.f;
    for (int m = 0; m < gs; ++m) {
      const float x = q_l[g * D + t * gs + m];
      e += x * x;
    }
    qe_l[i] = e;
  }
  __syncthreads();

  const int grp8 = lane >> 3, j = lane & 7;
  const int vpart = lane / LPBV, vq = lane % LPBV;
  const float4* kbar4 = reinterpret_cast<const float4*>(a.kbar);
  const float4* vbar4 = reinterpret_cast<const float4*>(a.vbar);
  const float4* q4 = reinterpret_cast<const float4*>(q_l);
  const size_t ubase = (size_t)unit * a.cap_blocks;
  float* uo = a.u + (size_t)unit * a.max_blocks * G;
  float* go = a.grp + (size_t)unit * a.NG * G * 2;
  const float invd = 1.0f / (float)D;
  const bool rvec = (r % 32) == 0;

  float mz[G], lz[G], acc[G][4];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    mz[g] = -INFINITY;
    lz[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[g][e] = 0.f;
  }

  const int c0 = chunk * a.BPC;
  const int c1 = min(c0 + a.BPC, NB);
  for (int base = c0 + wave * kBlocksPerWave; base < c1; base += kBlocksPerIter) {
    const int b0 = base + grp8, b1 = base + 8 + grp8;
    const bool v0 = b0 < c1, v1 = b1 < c1;
    // ---- loads: k̄ (8 lanes per block, coalesced 128 B rows), D̄, |b|, v̄
    float4 k0[KC], k1[KC];
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      k0[i] = v0 ? kbar4[(ubase + b0) * (D / 4) + j + 8 * i] : make_float4(0.f, 0.f, 0.f, 0.f);
      k1[i] = v1 ? kbar4[(ubase + b1) * (D / 4) + j + 8 * i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float4 d0[4], d1[4];
    float ds0[2], ds1[2];
    if (rvec) {
      const int RV = r / 32;
      const float4* dbar4 = reinterpret_cast<const float4*>(a.dbar);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = i < RV;
        d0[i] = (ok && v0) ? dbar4[(ubase + b0) * (r / 4) + j + 8 * i] : make_float4(0.f, 0.f, 0.f, 0.f);
        d1[i] = (ok && v1) ? dbar4[(ubase + b1) * (r / 4) + j + 8 * i] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    } else {
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2) {
        const int t = j + 8 * m2;
        ds0[m2] = (t < r && v0) ? a.dbar[(ubase + b0) * r + t] : 0.f;
        ds1[m2] = (t < r && v1) ? a.dbar[(ubase + b1) * r + t] : 0.f;
      }
    }
    const float n0 = v0 ? a.cnt[ubase + b0] : 1.f;
    const float n1 = v1 ? a.cnt[ubase + b1] : 1.f;
    float4 vv[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int bv = base + k * BPIV + vpart;
      vv[k] = bv < c1 ? vbar4[(ubase + bv) * (D / 4) + vq] : make_float4(0.f, 0.f, 0.f, 0.f);
    }

    // ---- z̄ and σ̂² (partial over the lane's coordinates, then over the 8 lanes)
    float z0[G], z1[G], s0[G], s1[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float za = 0.f, zb = 0.f;
#pragma unroll
      for (int i = 0; i < KC; ++i) {
        const float4 qq = q4[(g * D) / 4 + j + 8 * i];
        za += dot4(k0[i], qq);
        zb += dot4(k1[i], qq);
      }
      float sa = 0.f, sb = 0.f;
      if (rvec) {
        const int RV = r / 32;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i < RV) {
            const float4 e4 = reinterpret_cast<const float4*>(qe_l + g * r)[j + 8 * i];
            sa += dot4(d0[i], e4);
            sb += dot4(d1[i], e4);
          }
        }
      } else {
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2) {
          const int t = j + 8 * m2;
          const float e = t < r ? qe_l[g * r + t] : 0.f;
          sa += e * ds0[m2];
          sb += e * ds1[m2];
        }
      }
      z0[g] = xsum<1, 8>(za) * a.isd;
      z1[g] = xsum<1, 8>(zb) * a.isd;
      s0[g] = xsum<1, 8>(sa) * invd;
      s1[g] = xsum<1, 8>(sb) * invd;
    }

    // ---- scoring partials of this 16-block group
    const float ln0 = __logf(n0), ln1 = __logf(n1);
    const int gi = base / kBlocksPerWave;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float a0 = v0 ? ln0 + z0[g] + 0.5f * s0[g] : -INFINITY;
      const float a1 = v1 ? ln1 + z1[g] + 0.5f * s1[g] : -INFINITY;
      const float ref = xmax<8, 64>(fmaxf(a0, a1));
      const float e0 = v0 ? __expf(a0 - ref) : 0.f;
      const float e1 = v1 ? __expf(a1 - ref) : 0.f;
      const float l = xsum<8, 64>(e0 + e1);
      if (j == g) {
        if (v0) uo[(size_t)b0 * G + g] = e0 * s0[g];
        if (v1) uo[(size_t)b1 * G + g] = e1 * s1[g];
      }
      if (lane == g) {
        go[((size_t)gi * G + g) * 2] = ref;
        go[((size_t)gi * G + g) * 2 + 1] = l;
      }
    }

    // ---- Mean compensation of every block of the group (kept ones removed later)
    float* wl = w_l + wave * 16 * G;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float zm = xmax<8, 64>(fmaxf(v0 ? z0[g] : -INFINITY, v1 ? z1[g] : -INFINITY));
      const float M = fmaxf(mz[g], zm);
      const float sc = rescale(mz[g], M);
      const float w0 = v0 ? n0 * __expf(z0[g] - M) : 0.f;
      const float w1 = v1 ? n1 * __expf(z1[g] - M) : 0.f;
      lz[g] = lz[g] * sc + xsum<8, 64>(w0 + w1);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[g][e] *= sc;
      mz[g] = M;
      if (j == 0) {
        wl[grp8 * G + g] = w0;
        wl[(8 + grp8) * G + g] = w1;
      }
    }
    wave_sync();
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int bl = k * BPIV + vpart;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float w = wl[bl * G + g];
        acc[g][0] += w * vv[k].x;
        acc[g][1] += w * vv[k].y;
        acc[g][2] += w * vv[k].z;
        acc[g][3] += w * vv[k].w;
      }
    }
    wave_sync();
  }

  // ---- chunk's compensation sums: combine lane groups, then waves
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[g][e] = xsum<LPBV, 64>(acc[g][e]);
  if (vpart == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e) cmb[(wave * G + g) * W + 2 + 4 * vq + e] = acc[g][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      cmb[(wave * G + g) * W] = mz[g];
      cmb[(wave * G + g) * W + 1] = lz[g];
    }
  }
  __syncthreads();
  float* co = a.comp + ((size_t)unit * a.C + chunk) * G * W;
  for (int idx = tid; idx < G * W; idx += kThreads) {
    const int g = idx / W, e = idx - g * W;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, cmb[(w * G + g) * W]);
    float val;
    if (e == 0) {
      val = M;
    } else {
      val = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) val += cmb[(w * G + g) * W + e] * rescale(cmb[(w * G + g) * W], M);
    }
    co[idx] = val;
  }

  if (!last_arriver(a.ctr + unit, a.C, &last)) return;
  select_tail<G>(a, unit, NB, lds);
}

hipError_t launch_score(int d, int G, const ScoreArgs& a, int U, size_t lds, hipStream_t st) {
  void* args[] = {(void*)&a};
  const void* f = nullptr;
#define CKNV_SCORE_CASE(DD, GG) \
  if (d == DD && G == GG) f = (const void*)score_kernel<DD, GG>;
  CKNV_SCORE_CASE(64, 1) CKNV_SCORE_CASE(64, 2) CKNV_SCORE_CASE(64, 4) CKNV_SCORE_CASE(64, 8)
  CKNV_SCORE_CASE(128, 1) CKNV_SCORE_CASE(128, 2) CKNV_SCORE_CASE(128, 4) CKNV_SCORE_CASE(128, 8)
#undef CKNV_SCORE_CASE
  if (!f) return hipErrorInvalidValue;
  return hipLaunchKernel(f, dim3(U * a.C), dim3(kThreads), args, lds, st);
}

}  // namespace cknv
