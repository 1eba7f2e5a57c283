// Device helpers shared by the attention kernels: the running softmax state
// of a wave, the BF16 token tile of one 16-token block and its exact-plus-
// compensation update with the logits on MFMA, and partial-record merging.
// Internal to libcknv.
#pragma once

#include "cknv_internal.h"

namespace cknv {


// Running softmax state of one wave for the G query heads. Lane l owns value
// coordinates [l*VPL, l*VPL+VPL) (VPL = d/64) summed over every token it has
// absorbed; m and l are wave-uniform.
template <int D, int G>
struct WaveState {
  static constexpr int VPL = D / 64;
  float m[G], l[G], acc[G][VPL];
  __device__ void init() {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = -INFINITY;
      l[g] = 0.f;
#pragma unroll
      for (int e = 0; e < VPL; ++e) acc[g][e] = 0.f;
    }
  }
};

// Mean-compensation inputs of one kept block (to be subtracted): the lane's
// VPL coordinates of k̄ and v̄, and |b|.
template <int D>
struct BlockMean {
  static constexpr int VPL = D / 64;
  float kb[VPL], vb[VPL], n;
  float on;  // 1: the block removes its compensation, 0: it removes none
  __device__ void load(const float* kbar_row, const float* vbar_row, const float* cnt, int lane) {
#pragma unroll
    for (int e = 0; e < VPL; ++e) {
      kb[e] = kbar_row[lane * VPL + e];
      vb[e] = vbar_row[lane * VPL + e];
    }
    n = *cnt;
    on = 1.f;
  }
  // n, or 0 where the block removes nothing: a product, not a select, so
  // that the load of n stays unconditional and is waited for at use (a
  // select lets the compiler move the load under the condition and wait for
  // it, and everything issued before it, right there)
  __device__ __forceinline__ float mass() const { return n * on; }
};

// ---------------------------------------------------------------- MFMA tiles
// The logits of a 16-token tile on the matrix cores: S[t][g] = K[t] . q_g as
// v_mfma_f32_16x16x32_bf16 with A = the tile's keys (token t = row) and
// B = the query heads (head g = column, G of 16 used). The operand layouts
// (checked on gfx950): A lane l holds row l%16, k = 8*(l/16) + e; B lane l
// holds column l%16, the same k; D lane l holds column l%16, rows
// 4*(l/16) + e. The k index is mapped to key coordinates so that lane l reads
// D/4 consecutive coordinates of its token: instruction i, lane group
// c = l/16, element e -> coordinate (D/4)*c + 8*i + e (A and B agree, so the
// sum is the same). q is FP32: it goes in as two BF16 halves (q = hi + lo up
// to 2^-16 relative), and the BF16 keys are exact, so the logits carry
// FP32-level error. Softmax and the value sums stay on the vector units.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

template <int D>
struct TileM {
  static constexpr int NI = D / 32, VPL = D / 64;
  u32x4_t k[NI];   // keys, MFMA A layout
  uint32_t v[16];  // values: lane's VPL coordinates of every token (as Tile)
  int nt;          // valid tokens
  // NT: non-temporal loads (a streaming pass) or plain ones (a latency-bound gather).
  // All 16 token rows of the block are read (they lie inside the cache, the
  // block being below its capacity); rows at or past T hold anything and are
  // masked at use. One base address per lane then serves every load (the
  // rows are immediate offsets), which keeps two tiles' addresses out of the
  // registers.
  template <bool NT = false>
  __device__ void load(const uint16_t* kc, const uint16_t* vc, long tok0, long T, int lane) {
    const long left = T - tok0;
    nt = left <= 0 ? 0 : (left >= 16 ? 16 : (int)left);
    const int t = lane & 15, c = lane >> 4;
    const uint16_t* ks = kc + (size_t)(tok0 + t) * D + (D / 4) * c;
#pragma unroll
    for (int i = 0; i < NI; ++i) k[i] = ldg<NT>(reinterpret_cast<const u32x4_t*>(ks + 8 * i));
    const uint16_t* vs = vc + (size_t)tok0 * D + lane * VPL;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      v[j] = VPL == 2 ? stream_load_u1<NT>(vs + j * D) : stream_load_h<NT>(vs + j * D);  // masked at use
  }
};

// The query heads as MFMA B operands (head l%16 < G, zero columns after).
// Lane l needs q of head l%16 at coordinates (D/4)*(l/16) + 8i + e: D/4
// consecutive floats, read from a padded LDS copy (below). From the plain
// [G][D] layout every such read falls on one bank (a conflict per
// instruction of about 1.5 us per wave); from global memory each wave's
// 8 KB of reads share the L1 path with its tile's loads. fetch_lds issues
// the LDS reads; build_from converts once they have arrived.
template <int D>
struct QMfma {
  static constexpr int NI = D / 32;
  bf16x8_t hi[NI], lo[NI];
  struct Raw {
    float4 x[NI][2];
  };
  // An LDS copy of q to build the operand from: head h's quarter c
  // (coordinates (D/4)c ..) at word h*kRowStride + c*kQuarterStride. The
  // strides (row = 16 words mod 32, quarter = 4 words mod 32) spread the
  // (head, quarter) pieces a wave reads at once over the banks: at 4 heads
  // at most two share a bank group (the unpadded [G][D] layout puts all of
  // them in one).
  static constexpr int kQuarterStride = D / 4 + 4;
  static constexpr int kRowStride = 4 * kQuarterStride;
  template <int G>
  static constexpr int lds_words() { return G * kRowStride; }
  // thread t < G*D/4: float4 t of the G heads (head t/(D/4)) into the copy
  __device__ static void stage(float* qm, int t, float4 v) {
    const int h = t / (D / 4), f = t - h * (D / 4);
    const int c = f / (D / 16), o = 4 * f - c * (D / 4);
    *reinterpret_cast<float4*>(qm + h * kRowStride + c * kQuarterStride + o) = v;
  }
  template <int G>
  __device__ static Raw fetch_lds(const float* qm, int lane) {
    const int j = lane & 15, c = lane >> 4;
    const float4* src = reinterpret_cast<const float4*>(qm + (j < G ? j : 0) * kRowStride + c * kQuarterStride);
    Raw r;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      r.x[i][0] = src[2 * i];
      r.x[i][1] = src[2 * i + 1];
    }
    return r;
  }
  template <int G>
  __device__ void build_from(const Raw& r, int lane) {
    const float keep = (lane & 15) < G ? 1.f : 0.f;  // columns past the G heads are zero
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const float v[8] = {r.x[i][0].x, r.x[i][0].y, r.x[i][0].z, r.x[i][0].w,
                          r.x[i][1].x, r.x[i][1].y, r.x[i][1].z, r.x[i][1].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = v[e] * keep;
        const __bf16 h = (__bf16)x;
        hi[i][e] = h;
        lo[i][e] = (__bf16)(x - (float)h);
      }
    }
  }
};

__device__ __forceinline__ float lane_value(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// absorb<D, G, COMP> with the logits on MFMA: add one block's exact terms and
// (COMP) remove its compensation terms (none when bm.mass() = 0). `pw`: this wave's LDS
// scratch of 16*G floats (the probabilities, read back as broadcasts).
template <int D, int G, bool COMP = true>
__device__ __forceinline__ void absorb_mfma(WaveState<D, G>& st, const TileM<D>& t, const BlockMean<D>& bm,
                                            const QMfma<D>& qm, const float* q_l, float* pw, int lane,
                                            float isd) {
  constexpr int VPL = D / 64, NI = D / 32;
  static_assert(G <= 16, "one MFMA column per query head");
  const int j = lane & 15, c = lane >> 4;
  float zbar[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    zbar[g] = -INFINITY;
    if constexpr (COMP) {
      float zp = 0.f;
#pragma unroll
      for (int e = 0; e < VPL; ++e) zp += bm.kb[e] * q_l[g * D + lane * VPL + e];
      zbar[g] = group_sum<64>(zp) * isd;
    }
  }
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const bf16x8_t a = __builtin_bit_cast(bf16x8_t, t.k[i]);
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qm.hi[i], s, 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qm.lo[i], s, 0, 0, 0);
  }
  float z[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) z[e] = 4 * c + e < t.nt ? s[e] * isd : -INFINITY;
  const float cmax = rows_max(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));  // head j's block max
  float M[G], sc[G], w[G];
  float Mj = -INFINITY;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float bmax = lane_value(cmax, g);
    if (COMP && bm.mass() > 0.f) bmax = fmaxf(bmax, zbar[g]);
    M[g] = fmaxf(st.m[g], bmax);
    sc[g] = rescale(st.m[g], M[g]);
    w[g] = COMP && bm.mass() > 0.f ? bm.mass() * __expf(zbar[g] - M[g]) : 0.f;
    Mj = j == g ? M[g] : Mj;
  }
  float p[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) p[e] = z[e] == -INFINITY ? 0.f : __expf(z[e] - Mj);
  const float ps = rows_sum((p[0] + p[1]) + (p[2] + p[3]));
  if (j < G) {
#pragma unroll
    for (int e = 0; e < 4; ++e) pw[(4 * c + e) * G + j] = p[e];
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    st.l[g] = st.l[g] * sc[g] + lane_value(ps, g) - w[g];
    st.m[g] = M[g];
#pragma unroll
    for (int e = 0; e < VPL; ++e) st.acc[g][e] *= sc[g];
  }
  // The wave reads back what its lanes just wrote (the fence keeps the
  // compiler from moving the reads ahead of the writes; the wave's LDS
  // operations then run in program order), four tokens at a time: LDS reads
  // do not move across the groups, so at most 4*G probabilities are held at
  // once.
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
  for (int t4 = 0; t4 < 16; t4 += 4) {
    if (t4 > 0) __builtin_amdgcn_sched_barrier(0x7F);  // ALU and global memory may cross, LDS may not
#pragma unroll
    for (int tk = t4; tk < t4 + 4; ++tk) {
      float pv[G];
#pragma unroll
      for (int g = 0; g < G; ++g) pv[g] = pw[tk * G + g];
      // tokens past nt may hold anything: their values are masked here, at
      // use, so that the tile's loads need not complete when issued
      const uint32_t vw = tk < t.nt ? t.v[tk] : 0u;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        st.acc[g][0] += pv[g] * bf16_lo(vw);
        if (VPL == 2) st.acc[g][1 % VPL] += pv[g] * bf16_hi(vw);
      }
    }
  }
  // the next tile's probability writes must not pass these reads
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  if constexpr (COMP) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < VPL; ++e) st.acc[g][e] -= w[g] * bm.vb[e];
  }
}

// Write the wave's record [m, l, 0, 0, acc[D]] per g.
template <int D, int G>
__device__ __forceinline__ void store_wave_record(const WaveState<D, G>& st, float* rec, int lane) {
  constexpr int VPL = D / 64, W = rec_words(D);
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < VPL; ++e) rec[g * W + 4 + lane * VPL + e] = st.acc[g][e];
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      rec[g * W] = st.m[g];
      rec[g * W + 1] = st.l[g];
      rec[g * W + 2] = 0.f;
      rec[g * W + 3] = 0.f;
    }
  }
}

// Per query head g of n records (LDS, G x W words each): M = max of m_i,
// the factors e^{m_i - M} into scl[i*G + g], and L = sum_i l_i e^{m_i - M}
// (starting from a running (M0, L0), whose factor goes to *s0).
template <int D, int G>
__device__ __forceinline__ void record_scales(const float* recs, int n, int g, float* scl, float& M,
                                              float& L, float* s0) {
  constexpr int W = rec_words(D);
  float MM = M;
  for (int i = 0; i < n; ++i) MM = fmaxf(MM, recs[(i * G + g) * W]);
  const float so = rescale(M, MM);
  float LL = L * so;
  for (int i = 0; i < n; ++i) {
    const float f = rescale(recs[(i * G + g) * W], MM);
    scl[i * G + g] = f;
    LL += recs[(i * G + g) * W + 1] * f;
  }
  if (s0) *s0 = so;
  M = MM;
  L = LL;
}

// sum_i recs[i][g][4 + c] * scl[i][g] over n records, four at a time.
template <int D, int G>
__device__ __forceinline__ float record_column(const float* recs, const float* scl, int n, int g, int c) {
  constexpr int W = rec_words(D);
  float A = 0.f;
  int i = 0;
#pragma unroll 1
  for (; i + 4 <= n; i += 4) {
    float x[4], f[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[k] = recs[((i + k) * G + g) * W + 4 + c];
      f[k] = scl[(i + k) * G + g];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) A += x[k] * f[k];
  }
  for (; i < n; ++i) A += recs[(i * G + g) * W + 4 + c] * scl[i * G + g];
  return A;
}

// Merge n records of G x W words (LDS, consecutive) into one record at dst
// (global). `scl` is LDS scratch of n*G floats. COHERENT: agent-scope stores
// (coherent across XCDs for a reader in another workgroup of this launch).
template <int D, int G, int NT = kThreads, bool COHERENT = false>
__device__ __forceinline__ void merge_records(const float* recs, int n, float* dst, float* scl) {
  constexpr int W = rec_words(D);
  const int tid = threadIdx.x;
  auto st = [](float* p, float v) {
    if constexpr (COHERENT) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *p = v;
  };
  if (tid < G) {
    float M = -INFINITY, L = 0.f;
    record_scales<D, G>(recs, n, tid, scl, M, L, nullptr);
    st(dst + tid * W, M);
    st(dst + tid * W + 1, L);
    st(dst + tid * W + 2, 0.f);
    st(dst + tid * W + 3, 0.f);
  }
  lds_barrier();
  for (int col = tid; col < G * D; col += NT) {
    const int g = col / D, c = col - g * D;
    st(dst + g * W + 4 + c, record_column<D, G>(recs, scl, n, g, c));
  }
}

// Merge N records of G x W words (LDS, consecutive) into one record at dst
// (global), with no barrier: each thread forms its columns' scale factors
// e^{m_i - M} itself (the m_i reads are broadcasts within a wave, whose
// columns lie in one query head). Query head g's (m, l) is also written as
// one float pair at hdr + 2*g*hstride. COHERENT: agent-scope stores, as
// merge_records.
template <int D, int G, int NT, int N, bool COHERENT>
__device__ __forceinline__ void merge_wave_records(const float* recs, float* dst, float* hdr, int hstride) {
  constexpr int W = rec_words(D), CW = (G * D + NT - 1) / NT;  // columns per thread
  static_assert(G * D % NT == 0 || CW == 1, "every thread owns CW columns");
  auto st = [](float* p, float v) {
    if constexpr (COHERENT) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *p = v;
  };
  if (CW == 1 && (int)threadIdx.x >= G * D) return;
  // every LDS read of every column first
  float m[CW][N], l[CW][N], x[CW][N];
#pragma unroll
  for (int k = 0; k < CW; ++k) {
    const int col = threadIdx.x + NT * k, g = col / D, c = col - g * D;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      m[k][i] = recs[(i * G + g) * W];
      l[k][i] = recs[(i * G + g) * W + 1];
      x[k][i] = recs[(i * G + g) * W + 4 + c];
    }
  }
#pragma unroll
  for (int k = 0; k < CW; ++k) {
    const int col = threadIdx.x + NT * k, g = col / D, c = col - g * D;
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < N; ++i) M = fmaxf(M, m[k][i]);
    float A = 0.f, L = 0.f;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const float f = rescale(m[k][i], M);
      A += x[k][i] * f;
      L += l[k][i] * f;
    }
    st(dst + g * W + 4 + c, A);
    if (c == 0) {
      st(dst + g * W, M);
      st(dst + g * W + 1, L);
      st(dst + g * W + 2, 0.f);
      st(dst + g * W + 3, 0.f);
      uint64_t* h = reinterpret_cast<uint64_t*>(hdr) + (size_t)g * hstride;
      const uint64_t bits = (uint64_t)__float_as_uint(M) | ((uint64_t)__float_as_uint(L) << 32);
      if constexpr (COHERENT) __hip_atomic_store(h, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else *h = bits;
    }
  }
}

template <int G>
constexpr int stage_cap() { return G <= 4 ? 24 : 12; }

// Copy n <= stage_cap records (G x W words each, 16-byte aligned) from global
// to LDS; every load is issued before the first LDS store.
template <int D, int G, int NT = kThreads>
__device__ __forceinline__ void stage_records(const float* src, int n, float* lds_dst) {
  constexpr int W4 = rec_words(D) / 4;
  constexpr int NBUF = (stage_cap<G>() * G * W4 + NT - 1) / NT;
  const float4* s4 = reinterpret_cast<const float4*>(src);
  float4* d4 = reinterpret_cast<float4*>(lds_dst);
  const int total = n * G * W4;
  float4 buf[NBUF];
#pragma unroll
  for (int k = 0; k < NBUF; ++k) {
    const int i = threadIdx.x + k * NT;
    buf[k] = i < total ? s4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int k = 0; k < NBUF; ++k) {
    const int i = threadIdx.x + k * NT;
    if (i < total) d4[i] = buf[k];
  }
}

// Merge a unit's P <= RB part records (RB <= 64) into out and lse, one
// output column per thread (columns tid + NT*k, k < COLS). The 64 columns of
// a wave lie in one query head, so the records' (m, l) are loaded once per
// wave, lane i holding record i's, and each record's weight e^{m_i - M}
// reaches the lanes by readlane: P + 1 loads per thread instead of 3P. The
// pairs come from `hdr` ([G][P] float pairs, parts contiguous: a wave's pair
// load touches 4 cache lines, where the records' own headers, a record
// apart, touch 64; the lines a merge requests, not its round trips, bound
// it). Every load is issued before the first use, the pair first (the
// reductions wait only for it). Slots past P reload record P - 1 with
// weight 0. COHERENT: agent-scope loads, as merge_parts.
template <int D, int G, int NT, int COLS, int RB, bool COHERENT>
__device__ __forceinline__ void merge_parts_lanes(const float* parts, const float* hdr, int P, float* out,
                                                  float* lse) {
  constexpr int W = rec_words(D);
  static_assert(D % 64 == 0, "a wave's columns lie in one head");
  static_assert(RB <= 64, "one record per lane");
  static_assert(G * D % NT == 0 || COLS == 1, "every thread owns COLS columns");
  const int tid = threadIdx.x, lane = tid & 63;
  auto ld = [](const float* p) {
    if constexpr (COHERENT) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else return *p;
  };
  if (tid - lane >= G * D) return;  // (COLS == 1 only) a wave with no column
  const int li = lane < P ? lane : P - 1;
  // every load of every column first: the pairs, then the columns' values
  float ml[COLS], ll[COLS], x[COLS][RB];
#pragma unroll
  for (int k = 0; k < COLS; ++k) {
    const int g = (tid + NT * k) / D;
    const uint64_t* hp = reinterpret_cast<const uint64_t*>(hdr) + (size_t)g * P + li;
    uint64_t mlb;
    if constexpr (COHERENT) mlb = __hip_atomic_load(hp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else mlb = *hp;
    ml[k] = __uint_as_float((uint32_t)mlb);
    ll[k] = __uint_as_float((uint32_t)(mlb >> 32));
  }
#pragma unroll
  for (int k = 0; k < COLS; ++k) {
    const int col = tid + NT * k, g = col / D, c = col - g * D;
    const float* pg = parts + (size_t)g * W;
#pragma unroll
    for (int t = 0; t < RB; ++t) x[k][t] = ld(pg + (size_t)(t < P ? t : P - 1) * G * W + 4 + c);
  }
#pragma unroll
  for (int k = 0; k < COLS; ++k) {
    const int col = tid + NT * k, g = col / D, c = col - g * D;
    const float mb = ml[k] + (lane < P ? 0.f : -INFINITY);
    const float M = group_max<64>(mb);
    const float f = rescale(mb, M);  // 0 past the last record
    const float L = group_sum<64>(ll[k] * f);
    float A = 0.f;
#pragma unroll
    for (int t = 0; t < RB; ++t) A += x[k][t] * __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), t));
    const bool ok = L > 0.f;
    out[col] = ok ? A / L : 0.f;
    if (c == 0 && lse) lse[g] = ok ? M + __logf(L) : -INFINITY;
  }
}

// Merge a unit's P part records into out and lse. Thread t owns output
// columns col0 + t + NT*k (k < COLS); records are read in batches of PB,
// every load of a batch issued before the first use. COHERENT: agent-scope
// loads (records written by other workgroups of the same launch with
// agent-scope stores).
template <int D, int G, int NT, int PB, int COLS, bool COHERENT>
__device__ __forceinline__ void merge_parts(const float* parts, int P, float* out, float* lse, int col0) {
  constexpr int W = rec_words(D);
  const int tid = threadIdx.x;
  auto ld = [](const float* p) {
    if constexpr (COHERENT) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else return *p;
  };
  float M[COLS], L[COLS], A[COLS];
#pragma unroll
  for (int k = 0; k < COLS; ++k) { M[k] = -INFINITY; L[k] = 0.f; A[k] = 0.f; }
  for (int p0 = 0; p0 < P; p0 += PB) {
    float m[PB][COLS], l[PB][COLS], x[PB][COLS];
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int pi = p0 + i < P ? p0 + i : P - 1;
#pragma unroll
      for (int k = 0; k < COLS; ++k) {
        int col = col0 + tid + k * NT;
        col = col < G * D ? col : G * D - 1;
        const int g = col / D, c = col - g * D;
        const float* r = parts + ((size_t)pi * G + g) * W;
        m[i][k] = p0 + i < P ? ld(r) : -INFINITY;
        l[i][k] = ld(r + 1);
        x[i][k] = ld(r + 4 + c);
      }
    }
#pragma unroll
    for (int k = 0; k < COLS; ++k) {
      float MM = M[k];
#pragma unroll
      for (int i = 0; i < PB; ++i) MM = fmaxf(MM, m[i][k]);
      const float so = rescale(M[k], MM);
      float LL = L[k] * so, AA = A[k] * so;
#pragma unroll
      for (int i = 0; i < PB; ++i) {
        const float f = rescale(m[i][k], MM);
        LL += l[i][k] * f;
        AA += x[i][k] * f;
      }
      M[k] = MM;
      L[k] = LL;
      A[k] = AA;
    }
  }
#pragma unroll
  for (int k = 0; k < COLS; ++k) {
    const int col = col0 + tid + k * NT;
    if (col < G * D) {
      const bool ok = L[k] > 0.f;
      out[col] = ok ? A[k] / L[k] : 0.f;
      if (col % D == 0 && lse) lse[col / D] = ok ? M[k] + __logf(L[k]) : -INFINITY;
    }
  }
}

// A part of a unit counts itself done once its record's agent-scope stores
// are complete (the caller waits for them and holds a barrier first); true
// for the part that completes the unit's count. `uc`: the unit's counter,
// followed by its group counters. Up to kFlatParts parts count on the
// unit's counter; past that, on their group's (kPartGroup parts), whose
// last part resets it and counts the group in on the unit's (same-address
// atomics serialise). One thread calls this.
__device__ __forceinline__ bool count_part_in(uint32_t* uc, int p, int P) {
  auto count_in = [](uint32_t* c) {
    return __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  if (P <= kFlatParts) return count_in(uc) == (uint32_t)(P - 1);
  // the group's last part counts the group in (its own stores, and so those
  // of every part that counted into the group before it, are complete), and
  // resets the group's counter: no part of the group counts again
  const int grp = p / kPartGroup, ng = (P + kPartGroup - 1) / kPartGroup;
  const int gsize = P - grp * kPartGroup < kPartGroup ? P - grp * kPartGroup : kPartGroup;
  if (count_in(uc + 1 + grp) != (uint32_t)(gsize - 1)) return false;
  __hip_atomic_store(uc + 1 + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return count_in(uc) == (uint32_t)(ng - 1);
}

// The completing part's merge of a unit's P part records (`parts`, G x W
// words each; `hdr`: their (m, l) pairs, [G][P]) into out and lse, read with
// agent-scope loads: 1-64 parts by the lane merge, one straight-line
// instance per size class so that every load is issued before the first
// wait; more in batches of 8 records.
template <int D, int G, int NT>
__device__ __forceinline__ void merge_parts_any(const float* parts, const float* hdr, int P, float* out, float* lse) {
  constexpr int COLS = (G * D + NT - 1) / NT;
  if (P > 64)
    merge_parts<D, G, NT, 8, COLS, true>(parts, P, out, lse, 0);
  else if (P <= 8)
    merge_parts_lanes<D, G, NT, COLS, 8, true>(parts, hdr, P, out, lse);
  else if (P <= 16)
    merge_parts_lanes<D, G, NT, COLS, 16, true>(parts, hdr, P, out, lse);
  else if (P <= 32)
    merge_parts_lanes<D, G, NT, COLS, 32, true>(parts, hdr, P, out, lse);
  else
    merge_parts_lanes<D, G, NT, COLS, 64, true>(parts, hdr, P, out, lse);
}

}  // namespace cknv
