// Projection GEMMs of the drafter: out[s][m][n] = sum_{k in split s} A[m,k] * W[n,k].
//
// For the bf16 storage type W is fp16 in the fragment-packed layout (packed
// once from the caller's bf16 matrices, see pack_weight_k below) and streams
// from HBM once; A is an fp32 activation or the caller's bf16 features, both
// rounded to fp16 where they enter the matrix cores (single pass, fp32
// accumulation).  The fp32 storage type runs a plain fp32 kernel.
//
// Three kernels, chosen by shape:
//  * skinny (M <= 64): weight streaming.  Workgroup w (four waves) owns K split
//    s = w % S and the 64-column tiles w / S, w / S + wps, ... (wps = workgroups
//    per split, ~256 workgroups in all).  Consecutive workgroups thus read the S
//    slices of the same tiles, so at any moment the chip streams a few
//    contiguous regions of the packed weight, which measured ~20% faster than
//    giving each workgroup a contiguous run of tiles.  A workgroup stages its
//    activation slice A[:, split] once in LDS (fp16, in MFMA fragment order,
//    RMSNorm folded in); each wave then streams the packed fragments of its 16
//    weight rows, 1 KB per load instruction, two register buffers of U k-steps
//    in flight across tile boundaries, into v_mfma_f32_16x16x32_f16.  At
//    M = batch*16 the arithmetic intensity is ~16 flop/B, far below the MFMA
//    ridge: the kernel is HBM-bound and the matrix cores only keep the FMA work
//    off the VALU.
//  * mfma (M > 64, a contraction): the activation rows are first written as
//    fp16 fragments in the weights' packed layout (pack_rows_k: RMSNorm folded
//    in, rows padded to 256), then 256x256 output tiles are computed by 8 waves
//    of 128x64 from v_mfma_f32_16x16x32_f16, both operands streamed into LDS by
//    direct-to-LDS 16-byte loads (each wave writes whole 1 KB fragments, already
//    in MFMA order) through a 3-stage pipeline with one barrier per 32-wide k
//    step; split K fills the 256 CUs when the tiles alone do not.
//  * f32: a plain LDS-tiled FMA kernel for the fp32 storage type.
// Partial sums over K splits are reduced, in split order, by the consumer
// kernel, which also applies the epilogue (residual, norm, RoPE, SwiGLU).

#include "common.h"
#include "kernels.h"
#include "mfma_tile.h"

namespace {

constexpr int SK_U = 8;            // k-steps (of 32) per prefetch buffer
constexpr int SK_WAVES = 4;
constexpr int SK_THREADS = 64 * SK_WAVES;
constexpr int SK_NT = 16 * SK_WAVES;  // output columns per item (16 per wave)
constexpr int SK_GRID = 256;       // one workgroup per CU

// A segment holding columns [k0, k0 + kc) of a K split (plan_gemm makes kc divide
// ka_w, so a split never straddles two segments), offset to column k0.  k0 must
// be uniform (scalar registers).
template <typename TA>
__device__ __forceinline__ const TA* a_split(const GemmArgs& g, int k0) {
  const int seg = k0 / g.ka_w;
  const void* a = g.a[0];
#pragma unroll
  for (int i = 1; i < DF_MAX_ASEG; ++i)
    if (seg == i) a = g.a[i];
  return (const TA*)a + (k0 - seg * g.ka_w);
}

// Packed fragment (16-row group c, k-step t) of the concatenated weight: lane l
// of the returned pointer + 8 l holds rows 16c + l%16, k = 32t + 8(l/16) .. +8.
// Groups past N map to group 0 (ok = false) so loads stay in bounds.  c must be
// wave-uniform: the segment search then runs on scalar registers and reads the
// kernel-argument arrays with scalar loads (a per-lane index would turn each
// lookup into a vector load of kernel-argument memory on the critical path).
__device__ __forceinline__ const f16_t* wfrag(const GemmArgs& g, int c, int t, bool& ok) {
  const int n = c * 16;
  ok = n < g.N;
  const int nn = ok ? n : 0;
  const void* w = g.w[0];
  int off = 0;
  if (g.n_wseg > 1 && nn >= g.n_off[1]) { w = g.w[1]; off = g.n_off[1]; }
  if (g.n_wseg > 2 && nn >= g.n_off[2]) { w = g.w[2]; off = g.n_off[2]; }
  if (g.n_wseg > 3 && nn >= g.n_off[3]) { w = g.w[3]; off = g.n_off[3]; }
  if (g.n_wseg > 4 && nn >= g.n_off[4]) {
    int j = 4;
    while (j + 1 < g.n_wseg && nn >= g.n_off[j + 1]) ++j;
    w = g.w[j];
    off = g.n_off[j];
  }
  return (const f16_t*)w + ((long long)((nn - off) >> 4) * (g.K >> 5) + t) * 512;
}

// srs[r] = 1 / RMS of A row r0 + r (r < n) from its partial sums of squares
// (the norm is folded into the A staging).  16 threads per row, each summing
// every 16th chunk with batched loads, then a 16-lane butterfly: all rows of a
// pass cost one memory latency.
template <int NTHREADS>
__device__ __forceinline__ void rows_rs(const GemmArgs& g, int r0, int n, float* srs) {
  const int sub = threadIdx.x & 15;
  for (int rb = 0; rb < n; rb += NTHREADS / 16) {
    const int r = rb + (int)(threadIdx.x >> 4);
    float t = 0.f;
    if (r < n && sub < g.nss_chunks)
      t = sum_strided(g.nss + (long long)(r0 + r) * g.nss_chunks + sub, 16,
                      (g.nss_chunks - sub + 15) / 16);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) t += __shfl_xor(t, o, 64);
    if (sub == 0 && r < n) srs[r] = rsqrtf(t / g.K + g.neps);
  }
}

// A fragment (8 consecutive k of one row) as fp16, from the split's segment
// base `ab` (column kk relative to the split start k0).  AF32: fp32 activation,
// scaled by rs * gain[k0 + kk] first when a norm is folded in; else bf16 features.
template <bool AF32>
__device__ __forceinline__ f16x8 load_a8(const GemmArgs& g, const void* ab, int row, int k0, int kk,
                                         float rs) {
  if (AF32) {
    const float* p = (const float*)ab + (long long)row * g.lda + kk;
    floatx4 a = *(const floatx4*)p, b = *(const floatx4*)(p + 4);
    if (g.nss) {
      const u32x4 gw = *(const u32x4*)((const bf16_t*)g.ngain + k0 + kk);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        a[2 * j] *= rs * __uint_as_float(gw[j] << 16);
        a[2 * j + 1] *= rs * __uint_as_float(gw[j] & 0xFFFF0000u);
        b[2 * j] *= rs * __uint_as_float(gw[2 + j] << 16);
        b[2 * j + 1] *= rs * __uint_as_float(gw[2 + j] & 0xFFFF0000u);
      }
    }
    return cvt8(a, b);
  }
  return bf8_to_h8(*(const u32x4*)((const bf16_t*)ab + (long long)row * g.lda + kk));
}

// Skinny GEMM: workgroup (split s = w % S, index wi = w / S) stages A[:, split s]
// once, then streams tiles wi, wi + wps, ... and stores fp32 partial sums into out[s].
template <int MT, bool AF32>
__global__ __launch_bounds__(SK_THREADS) void gemm_skinny(GemmArgs g) {
  extern __shared__ f16x8 sA[];  // [(t * MT + mt) * 64 + lane]
  __shared__ float srs[MT * 16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int s = blockIdx.x % g.S, wi = blockIdx.x / g.S;
  const int k0 = s * g.kc;
  const int T = g.kc / 32;
  const int nslots = T * MT * 64;
  const int ntiles = (g.N + SK_NT - 1) / SK_NT;
  const void* ab = AF32 ? (const void*)a_split<float>(g, k0) : (const void*)a_split<bf16_t>(g, k0);

  // this workgroup's tiles: wi, wi + wps, ... < ntiles; c = 16-row group of a wave
  const int n_my = (ntiles - wi + g.wps - 1) / g.wps;
  if (n_my <= 0) return;
  auto tile_ptr = [&](int j) {
    bool ok;
    return wfrag(g, (wi + j * g.wps) * SK_WAVES + wave, k0 >> 5, ok) + lane * 8;
  };
  f16x8 wa[SK_U];
  // slot (t, mt, l) = A[mt*16 + l%16][k0 + 32t + 8(l/16) ..+8]
  int p_rest = threadIdx.x;  // first slot still to stage
  if constexpr (MT == 1) {
    // One memory latency for the whole prologue: the row statistics' partial
    // sums, this thread's A slots and the first weight buffer are all requested
    // before any of them is waited for (loads complete in issue order, so the
    // weights go last).
    constexpr int PS = 8;  // slots per thread staged this way (kc <= 1024)
    const int rrow = threadIdx.x >> 4, sub = threadIdx.x & 15;
    // row statistics: 16 threads per row, up to SS_T chunks each (clamped,
    // unconditional loads; the invalid ones are dropped where summed)
    constexpr int SS_T = 32;
    float ssr[SS_T];
    if (AF32 && g.nss) {
      const float* sp = g.nss + (long long)min(rrow, g.M - 1) * g.nss_chunks;
#pragma unroll
      for (int c = 0; c < SS_T; ++c) ssr[c] = sp[min(sub + 16 * c, g.nss_chunks - 1)];
    }
    floatx4 ra[PS], rb[PS];
    u32x4 rg[PS];
#pragma unroll
    for (int j = 0; j < PS; ++j) {
      const int p = threadIdx.x + j * SK_THREADS;
      const int l = p & 63, t = p >> 6, row = l & 15;
      const int kk = t * 32 + (l >> 4) * 8;
      ra[j] = rb[j] = floatx4{0.f, 0.f, 0.f, 0.f};
      rg[j] = u32x4{0u, 0u, 0u, 0u};
      if (p < nslots && row < g.M) {
        if (AF32) {
          const float* ap = (const float*)ab + (long long)row * g.lda + kk;
          ra[j] = *(const floatx4*)ap;
          rb[j] = *(const floatx4*)(ap + 4);
          if (g.nss) rg[j] = *(const u32x4*)((const bf16_t*)g.ngain + k0 + kk);
        } else {
          rg[j] = *(const u32x4*)((const bf16_t*)ab + (long long)row * g.lda + kk);
        }
      }
    }
    load_w<SK_U>(wa, tile_ptr(0), 0);
    if (AF32 && g.nss) {
      float t = 0.f;  // invalid terms multiplied by 0 (a use on every path keeps each load early)
#pragma unroll
      for (int c = 0; c < SS_T; ++c) t += ssr[c] * (float)(rrow < g.M && sub + 16 * c < g.nss_chunks);
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) t += __shfl_xor(t, o, 64);
      if (sub == 0 && rrow < 16) srs[rrow] = rsqrtf(t / g.K + g.neps);
      barrier_after_lds_stores();
    }
#pragma unroll
    for (int j = 0; j < PS; ++j) {
      const int p = threadIdx.x + j * SK_THREADS;
      if (p >= nslots) break;
      const int row = p & 15;
      f16x8 v;
      if (AF32) {
        floatx4 a = ra[j], b = rb[j];
        if (g.nss) {
          const float rs = row < g.M ? srs[row] : 0.f;
          const u32x4 gw = rg[j];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            a[2 * q] *= rs * __uint_as_float(gw[q] << 16);
            a[2 * q + 1] *= rs * __uint_as_float(gw[q] & 0xFFFF0000u);
            b[2 * q] *= rs * __uint_as_float(gw[2 + q] << 16);
            b[2 * q + 1] *= rs * __uint_as_float(gw[2 + q] & 0xFFFF0000u);
          }
        }
        v = cvt8(a, b);
      } else {
        v = bf8_to_h8(rg[j]);
      }
      sA[p] = v;
    }
    p_rest = threadIdx.x + PS * SK_THREADS;
  } else {
    if (AF32 && g.nss) {
      rows_rs<SK_THREADS>(g, 0, min(g.M, MT * 16), srs);
      barrier_after_lds_stores();
    }
  }
#pragma unroll 4
  for (int p = p_rest; p < nslots; p += SK_THREADS) {
    const int l = p & 63;
    const int tm = p >> 6;
    const int mt = tm % MT, t = tm / MT;
    const int row = mt * 16 + (l & 15);
    f16x8 v = {};
    if (row < g.M)
      v = load_a8<AF32>(g, ab, row, k0, t * 32 + (l >> 4) * 8, (AF32 && g.nss) ? srs[row] : 1.f);
    sA[p] = v;
  }
  if constexpr (MT != 1) load_w<SK_U>(wa, tile_ptr(0), 0);
  barrier_after_lds_stores();

  float* out = g.out + (long long)s * g.M * g.N;
  stream_tiles<SK_U, MT>(n_my, T, tile_ptr, sA, lane, wa, [&](int j, const floatx4(&acc)[MT]) {
    const int n = ((wi + j * g.wps) * SK_WAVES + wave) * 16 + (lane & 15);
    if (n >= g.N) return;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = mt * 16 + (lane >> 4) * 4 + i;
        if (m < g.M) out[(long long)m * g.N + n] = acc[mt][i];
      }
    }
  });
}

// ---- full-K GEMMs for one 16-row group (M <= 16) --------------------------------
// One workgroup owns one 16-column output group (two for gate/up: gate group c and
// up group c) over the whole of K; its KW waves take equal slices of K, each
// streaming the packed weight and the packed fp16 A rows (L2-resident) one
// fragment per k step, and the slices are summed in LDS in wave order.  No
// partial sums leave the workgroup, so the epilogue finishes the output in place:
//   RK_RESID    X += A W^T, and the row statistics of the new X (ss_out);
//   RK_RESID_Y  as RK_RESID, and Y = fp16(X_new * gain * sc) as the next GEMM's
//               packed A rows, sc[m] = rsqrt(mean(X_old^2) + eps) from ss_in (the
//               statistics of X before the update: a per-row scale of the right
//               magnitude that every workgroup knows before the new norm exists);
//   RK_SWIGLU   g = (A Wg^T) r, u = (A Wu^T) r with r = rsqrt(mean(X^2) + eps) / sc
//               (ss_in: statistics of X, sc: the scale A was stored with), so that
//               A r is RMSNorm(X) * gain; writes silu(g) u as packed fp16 A rows.
//   RK_QKV      Q | K | V of the same normalised A (r as for RK_SWIGLU); a workgroup
//               owns the 16 dims i and the 16 dims i + d/2 of one head, so that it
//               applies RoPE itself: writes q rows and the block's K/V in the cache.
// KW waves split K; each keeps two register buffers of U k steps in flight.
// Measured on the 4096-wide batch-1 shapes: 4 waves with 8 k steps per buffer (one
// stream) or 4 (two streams) beat 8 waves and other buffer depths (QKV 13.2 us with
// 4 waves, 14.1 with 8; gate/up 32.4 with 4, 34.4 with 8).
enum RowkMode { RK_RESID, RK_RESID_Y, RK_SWIGLU, RK_QKV };
// (waves, k steps per buffer): one weight stream over K <= 4096 (output projection)
// or longer K (down projection), two streams (gate and up), and QKV
constexpr int RK_KW_S = 4, RK_U_S = 8;
constexpr int RK_KW_L = 4, RK_U_L = 8;
constexpr int RK_KW2 = 4, RK_U2 = 4;
constexpr int RK_KWQ = 4, RK_UQ = 4;
constexpr int RK_SSV = 8;

struct RowkArgs {
  const f16_t* A;  // packed fp16, one 16-row group, K columns
  const f16_t* W;  // packed [N][K] (gate for RK_SWIGLU)
  const f16_t* W2; // RK_SWIGLU: packed up [N][K]
  int M, N, K;
  float* X;             // RK_RESID*: fp32 rows [M][N], updated in place
  float* ss_out;        // RK_RESID*: [M][N / 16] chunk sums of squares of the new X
  const float* ss_in;   // RK_RESID_Y / RK_SWIGLU: [M][nch_in] chunk sums (see above)
  int nch_in;
  const bf16_t* gain;   // RK_RESID_Y: gain of the next RMSNorm, [N]
  float eps;
  float* sc;            // RK_RESID_Y writes [16], RK_SWIGLU reads
  f16_t* out16;         // RK_RESID_Y: Y; RK_SWIGLU: silu(g) u; packed, 16 rows, N columns
  // RK_QKV: packed Wq / Wk / Wv, the per-row (cos, sin) table [M][d/2], q rows
  // [M][Hq d], this layer's packed fp16 cache, rows m = b B + j at position len[b] + j
  const f16_t* Wv;
  const int32_t* len;
  const float* rope;
  float* q;
  f16_t* kc;
  f16_t* vc;
  int B, Hq, Hkv, d, max_ctx;
};

__device__ __forceinline__ int pk_index(int m, int k) {  // packed A, 16-row group 0
  return (((k >> 5) * 64) + m + 16 * ((k & 31) >> 3)) * 8 + (k & 7);
}

// Chunk sums of ss_in for rows 0..15 (clamped to M-1), this wave's share of the KW
// shares: lane l covers row l % 16, chunks [w (nch/KW) + (l/16) pl, + pl), pl = nch/(4 KW).
struct SsLoads {
  floatx4 v[RK_SSV];
};
template <int KW>
__device__ __forceinline__ void ss_issue(SsLoads& s, const float* ss, int M, int nch, int wave,
                                         int lane) {
  const int row = min(lane & 15, M - 1), pl = nch / (4 * KW);
  const float* b = ss + (long long)row * nch + wave * (nch / KW) + (lane >> 4) * pl;
#pragma unroll
  for (int j = 0; j < RK_SSV; ++j) s.v[j] = *(const floatx4*)(b + min(4 * j, pl - 4));
}
template <int KW>
__device__ __forceinline__ float ss_finish(const SsLoads& s, int nch) {
  const int pl = nch / (4 * KW);
  float t = 0.f;
#pragma unroll
  for (int j = 0; j < RK_SSV; ++j)
    t += (s.v[j][0] + s.v[j][1] + s.v[j][2] + s.v[j][3]) * (float)(4 * j < pl);
  t += __shfl_xor(t, 16, 64);
  t += __shfl_xor(t, 32, 64);
  return t;  // this wave's part of the row sum, row = lane % 16
}

template <int MODE, int KW, int U>
__global__ __launch_bounds__(KW * 64) void gemm_rowk(RowkArgs r) {
  constexpr int NW = MODE == RK_SWIGLU || MODE == RK_QKV ? 2 : 1;  // weight streams
  constexpr bool SSIN = MODE != RK_RESID;
  __shared__ floatx4 red[NW][KW][64];
  __shared__ float rpart[KW][16];
  const int c = blockIdx.x, lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int T = r.K / 32, tq = T / KW, t0 = wave * tq;
  SsLoads ssl;
  if constexpr (SSIN) ss_issue<KW>(ssl, r.ss_in, r.M, r.nch_in, wave, lane);
  // weight groups: c (and c of W2), or for RK_QKV dims j16.. and j16 + d/2.. of head hh
  const f16_t* w0 = r.W + (long long)c * T * 512;
  const f16_t* w1 = r.W2 + (long long)c * T * 512;
  int hh = 0, lh = 0, j16 = 0;
  if constexpr (MODE == RK_QKV) {
    const int gph = r.d / 32;  // 16-dim groups per half head
    hh = c / gph;
    j16 = (c % gph) * 16;
    const f16_t* seg = hh < r.Hq ? r.W : hh < r.Hq + r.Hkv ? r.W2 : r.Wv;
    lh = hh < r.Hq ? hh : hh < r.Hq + r.Hkv ? hh - r.Hq : hh - r.Hq - r.Hkv;
    w0 = seg + ((long long)lh * (r.d / 16) + c % gph) * T * 512;
    w1 = w0 + (long long)gph * T * 512;
  }
  const f16x8* wp[NW];
  wp[0] = (const f16x8*)(w0 + (long long)t0 * 512) + lane;
  if constexpr (NW == 2) wp[NW - 1] = (const f16x8*)(w1 + (long long)t0 * 512) + lane;
  const f16x8* ap = (const f16x8*)(r.A + (long long)t0 * 512) + lane;
  floatx4 acc[NW];
#pragma unroll
  for (int v = 0; v < NW; ++v) acc[v] = floatx4{0.f, 0.f, 0.f, 0.f};
  f16x8 wa[NW][U], aa[U], wb[NW][U], ab[U];
  auto load = [&](int t, f16x8 (&w)[NW][U], f16x8 (&a)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int v = 0; v < NW; ++v) w[v][u] = __builtin_nontemporal_load(wp[v] + (t + u) * 64);
      a[u] = ap[(t + u) * 64];
    }
  };
  auto mma = [&](const f16x8 (&w)[NW][U], const f16x8 (&a)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int v = 0; v < NW; ++v)
        acc[v] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[u], w[v][u], acc[v], 0, 0, 0);
  };
  // two register buffers in flight; the last pair is peeled so that the loop
  // body has no conditional load (its waits then count exactly)
  load(0, wa, aa);
  // The epilogue's own inputs (residual rows, next gain, row scales, rotation table,
  // sequence lengths; none is written by this kernel) are requested now, behind the
  // first weight buffer, so that no memory latency is left for the tail.  Every wave
  // issues them (no branch, so the loop's waits keep counting exactly), wave 0 uses
  // them; rows past M read row M - 1 and are discarded.
  const int n = c * 16 + (lane & 15);
  float xin[4] = {0.f, 0.f, 0.f, 0.f}, scin[4] = {0.f, 0.f, 0.f, 0.f};
  float csin[4] = {0.f, 0.f, 0.f, 0.f}, snin[4] = {0.f, 0.f, 0.f, 0.f};
  int lenin[4] = {0, 0, 0, 0};
  float gin = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = (lane >> 4) * 4 + i, mc = min(m, r.M - 1);
    if constexpr (MODE == RK_RESID || MODE == RK_RESID_Y) xin[i] = r.X[(long long)mc * r.N + n];
    if constexpr (MODE == RK_SWIGLU || MODE == RK_QKV) scin[i] = r.sc[m];
    if constexpr (MODE == RK_QKV) {
      const long long ro = ((long long)mc * (r.d >> 1) + j16 + (lane & 15)) * 2;
      csin[i] = r.rope[ro];
      snin[i] = r.rope[ro + 1];
      lenin[i] = r.len[mc / r.B];
    }
  }
  if constexpr (MODE == RK_RESID_Y) gin = bf2f(r.gain[n]);
  int t = 0;
  for (; t + 2 * U < tq; t += 2 * U) {  // tq is a multiple of 2 U
    load(t + U, wb, ab);
    __builtin_amdgcn_sched_barrier(0);
    mma(wa, aa);
    load(t + 2 * U, wa, aa);
    __builtin_amdgcn_sched_barrier(0);
    mma(wb, ab);
  }
  load(t + U, wb, ab);
  __builtin_amdgcn_sched_barrier(0);
  mma(wa, aa);
  mma(wb, ab);
#pragma unroll
  for (int v = 0; v < NW; ++v) red[v][wave][lane] = acc[v];
  if constexpr (SSIN) {
    const float part = ss_finish<KW>(ssl, r.nch_in);
    if (lane < 16) rpart[wave][lane] = part;
  }
  __syncthreads();
  if (wave != 0) return;
  floatx4 sum[NW];
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    sum[v] = red[v][0][lane];
#pragma unroll
    for (int w = 1; w < KW; ++w) sum[v] += red[v][w][lane];
  }
  // per-row factor from ss_in for the rows this lane holds (m = 4 (lane / 16) + i)
  float rowf[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (SSIN) {
    const float H_in = (float)(r.nch_in * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = (lane >> 4) * 4 + i;
      float tot = 0.f;
#pragma unroll
      for (int w = 0; w < KW; ++w) tot += rpart[w][m];
      rowf[i] = rsqrtf(tot / H_in + r.eps);
    }
  }
  if constexpr (MODE == RK_QKV) {
    const int half = r.d >> 1, di = j16 + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = (lane >> 4) * 4 + i;
      if (m >= r.M) continue;
      const float f = rowf[i] / scin[i];
      float y1 = sum[0][i] * f, y2 = sum[1][i] * f;
      if (hh < r.Hq + r.Hkv) {  // RoPE on the pair (di, di + d/2)
        const float cs = csin[i], sn = snin[i];
        const float x1 = y1, x2 = y2;
        y1 = x1 * cs - x2 * sn;
        y2 = x2 * cs + x1 * sn;
      }
      if (hh < r.Hq) {
        float* qo = r.q + (long long)m * r.Hq * r.d + hh * r.d;
        qo[di] = y1;
        qo[di + half] = y2;
        continue;
      }
      const int b = m / r.B, pos = lenin[i] + m % r.B;
      if (pos >= r.max_ctx) continue;
      const long long slice = ((long long)b * r.Hkv + lh) * r.max_ctx * r.d;
      if (hh < r.Hq + r.Hkv) {
        r.kc[slice + kfrag_off(pos, di, r.d)] = f2h(y1);
        r.kc[slice + kfrag_off(pos, di + half, r.d)] = f2h(y2);
      } else {
        r.vc[slice + vfrag_off(pos, di, r.d)] = f2h(y1);
        r.vc[slice + vfrag_off(pos, di + half, r.d)] = f2h(y2);
      }
    }
  } else if constexpr (MODE == RK_SWIGLU) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = (lane >> 4) * 4 + i;
      const float f = rowf[i] / scin[i];
      const float g = sum[0][i] * f, u = sum[NW - 1][i] * f;
      const float a = m < r.M ? g / (1.f + __expf(-g)) * u : 0.f;
      r.out16[pk_index(m, n)] = f2h(a);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = (lane >> 4) * 4 + i;
      float v = 0.f;
      if (m < r.M) {
        v = xin[i] + sum[0][i];
        r.X[(long long)m * r.N + n] = v;
      }
      if constexpr (MODE == RK_RESID_Y) {
        r.out16[pk_index(m, n)] = f2h(v * gin * rowf[i]);
        if (c == 0 && (lane & 15) == 0) r.sc[m] = rowf[i];
      }
      float s2 = v * v;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) s2 += __shfl_xor(s2, o, 64);
      if ((lane & 15) == 0 && m < r.M) r.ss_out[(long long)m * (r.N / 16) + c] = s2;
    }
  }
}

// ---- MFMA tiles (M > 64) -------------------------------------------------------
// Activation rows -> fp16 fragments in the packed layout (16-row groups x 32-wide
// k steps, 1 KB each), rows >= M zero.  Block (c, kb) handles row group c and
// k steps [8 kb, 8 kb + 8); with a folded norm, row r is scaled by rs[r] * gain.
template <bool AF32>
__global__ __launch_bounds__(256) void pack_rows_k(GemmArgs g) {
  __shared__ float srs[16];
  const int c = blockIdx.x;
  const int KT = g.K / 32;
  const int rows = min(16, g.M - 16 * c);
  if (AF32 && g.nss) {
    if (rows > 0) rows_rs<256>(g, 16 * c, rows, srs);
    __syncthreads();
  }
  const int t = blockIdx.y * 8 + (threadIdx.x >> 6) * 2;  // two k steps per wave
  const int l = threadIdx.x & 63;
  const int r = l & 15;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int tt = t + u;
    if (tt >= KT) break;
    const int k = 32 * tt;
    f16x8 v = {};
    if (r < rows) {
      const void* ab = AF32 ? (const void*)a_split<float>(g, k) : (const void*)a_split<bf16_t>(g, k);
      v = load_a8<AF32>(g, ab, 16 * c + r, k, (l >> 4) * 8, (AF32 && g.nss) ? srs[r] : 1.f);
    }
    *(f16x8*)(g.apack + (((long long)c * KT + tt) * 64 + l) * 8) = v;
  }
}

// out[s][m][n] over the TM x TN tile (mt, nt) and split s; tiles ordered row tile
// fastest, then column tile, then split, dealt to the XCDs by xcd_tile.  The
// SwiGLU epilogue (swiglu_out) runs on the 256 x 256 and 128 x 384 tiles: each wave's
// BG column groups are BG / 2 gate groups and the up groups of the same intermediate
// indices, TN / 2 of them per tile.
template <int TM, int TN>
__global__ __launch_bounds__(MF_WAVES * 64) void gemm_mfma(GemmArgs g, int n_mt, int n_nt,
                                                           int per_xcd) {
  using TL = MfTile<TM, TN>;
  constexpr int FPW = TL::FPW, FA = TL::FA, AG = TL::AG, BG = TL::BG;
  extern __shared__ f16x8 smem[];  // [MF_STG][FR fragments][64 lanes]: A groups, then B groups
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = xcd_tile(per_xcd);
  if (t >= n_mt * n_nt * g.S) return;
  const int mt = t % n_mt, nt = (t / n_mt) % n_nt, s = t / (n_mt * n_nt);
  const int KT = g.K / 32;
  const int kb = s * (g.kc / 32);
  const int nks = min(g.kc / 32, KT - kb);
  // this wave's fragments of a stage: f = wave * FPW + j (A group f, or B group f - FA)
  constexpr bool SW_TILE = (TM == 256 && TN == 256) || (TM == 128 && TN == 384);
  constexpr int HB = BG / 2;  // gate (and up) column groups of a wave
  const bool sw = SW_TILE && g.swiglu_out != nullptr;
  const f16_t* src[FPW];
#pragma unroll
  for (int j = 0; j < FPW; ++j) {
    const int f = wave * FPW + j;
    bool ok;
    const f16_t* p;
    if (f < FA) {
      p = g.apack + ((long long)(mt * FA + f) * KT + kb) * 512;
    } else if (sw) {
      // column group lg = BG wn + b of the tile: b < HB gate, b >= HB up, of the
      // 16 intermediate indices nt TN / 2 + 16 (HB wn + b % HB) ..
      const int lg = f - FA;
      const int b = lg % BG;
      const int grp = nt * (TN / 32) + (lg / BG) * HB + b % HB;
      p = (const f16_t*)g.w[b >= HB] + ((long long)grp * KT + kb) * 512;
    } else {
      p = wfrag(g, nt * (TN / 16) + f - FA, kb, ok);
    }
    src[j] = p + lane * 8;
  }
  floatx4 acc[AG][BG];
  mf_tile<TM, TN>(src, nks, smem, wave, lane, acc);
  const int wm = wave >> 2, wn = wave & 3;
  if constexpr (SW_TILE) {
    if (sw) {  // a[m][i] = silu(gate) * up, both halves in this wave's registers
      // element (m, i) of the packed fp16 A (K = I): fragment (m / 16, i / 32),
      // lane m % 16 + 16 ((i % 32) / 8), slot i % 8; rows >= M are left as they are
      // (their products land in output rows that are never stored)
      const int I = g.N / 2, IT = I / 32;
#pragma unroll
      for (int a = 0; a < AG; ++a)
#pragma unroll
        for (int j = 0; j < HB; ++j) {
          const int i = nt * (TN / 2) + (wn * HB + j) * 16 + (lane & 15);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = mt * TM + (AG * wm + a) * 16 + (lane >> 4) * 4 + r;
            const float gt = acc[a][j][r], up = acc[a][j + HB][r];
            if (m < g.M)
              g.swiglu_out[(((long long)(m >> 4) * IT + (i >> 5)) * 64 + (m & 15) + 16 * ((i & 31) >> 3)) * 8 +
                           (i & 7)] = f2h(gt / (1.f + __expf(-gt)) * up);
          }
        }
      return;
    }
  }
  float* out = g.out + (long long)s * g.M * g.N;
#pragma unroll
  for (int a = 0; a < AG; ++a)
#pragma unroll
    for (int b = 0; b < BG; ++b) {
      const int n = nt * TN + (BG * wn + b) * 16 + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = mt * TM + (AG * wm + a) * 16 + (lane >> 4) * 4 + r;
        if (m < g.M && n < g.N) out[(long long)m * g.N + n] = acc[a][b][r];
      }
    }
}

// ---- fp32 -----------------------------------------------------------------------
__global__ __launch_bounds__(256) void gemm_f32(GemmArgs g) {
  __shared__ float sA[16][33];
  __shared__ float sW[64][33];
  __shared__ float srs[16];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.y * 16, n0 = blockIdx.x * 64;
  if (g.nss) {
    rows_rs<256>(g, m0, min(16, g.M - m0), srs);
    __syncthreads();
  }
  const int s = blockIdx.z;
  const int col = tid & 63, rg = tid >> 6;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const int kbeg = s * g.kc, kend = kbeg + g.kc;
  for (int k0 = kbeg; k0 < kend; k0 += 32) {
    for (int p = tid; p < 16 * 32; p += 256) {
      const int r = p >> 5, c = p & 31;
      const int m = m0 + r, k = k0 + c;
      float v = 0.f;
      if (m < g.M) {
        v = a_split<float>(g, k0)[(long long)m * g.lda + c];  // 32 | segment width
        if (g.nss) v *= srs[r] * ((const float*)g.ngain)[k];
      }
      sA[r][c] = v;
    }
    for (int p = tid; p < 64 * 32; p += 256) {
      const int r = p >> 5, c = p & 31;
      const int n = n0 + r;
      float v = 0.f;
      if (n < g.N) {
        int j = 0;
        while (j + 1 < g.n_wseg && n >= g.n_off[j + 1]) ++j;
        v = ((const float*)g.w[j])[(long long)(n - g.n_off[j]) * g.ldw + k0 + c];
      }
      sW[r][c] = v;
    }
    __syncthreads();
#pragma unroll 8
    for (int c = 0; c < 32; ++c) {
      const float w = sW[col][c];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf(sA[rg * 4 + i][c], w, acc[i]);
    }
    __syncthreads();
  }
  const int n = n0 + col;
  if (n >= g.N) return;
  float* out = g.out + (long long)s * g.M * g.N;
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + rg * 4 + i;
    if (m < g.M) out[(long long)m * g.N + n] = acc[i];
  }
}

// Fragment-packed fp16 layout of a bf16 matrix W[N][K] (N % 16 == 0, K % 32 == 0):
// dst[((c * (K / 32) + t) * 64 + l) * 8 + j] = fp16(W[16 c + l % 16][32 t + 8 (l / 16) + j]),
// i.e. the B operand of v_mfma_f32_16x16x32_f16 for rows 16c.. and k-step t, so
// that one wave's 16-byte-per-lane load of a fragment is 1 KB contiguous.
// Elements that do not fit fp16 (converted to an infinity or NaN) are counted into
// *n_overflow (nullable).
__global__ __launch_bounds__(256) void pack_weight_k(const bf16_t* src, int N, int K, f16_t* dst,
                                                     int32_t* n_overflow) {
  const long long p = (long long)blockIdx.x * 256 + threadIdx.x;  // 16-byte piece of dst
  const long long npiece = (long long)N * K / 8;
  if (p >= npiece) return;
  const int l = (int)(p & 63);
  const long long ct = p >> 6;
  const int T = K / 32;
  const int c = (int)(ct / T), t = (int)(ct % T);
  const bf16_t* s = src + (long long)(16 * c + (l & 15)) * K + 32 * t + 8 * (l >> 4);
  const u32x4 v = *(const u32x4*)s;
  *(f16x8*)(dst + p * 8) = bf8_to_h8(v);
  int bad = 0;  // decided on the exact bf16 values: fp16 holds |x| < 65520 finitely
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    bad += !(fabsf(__uint_as_float(v[j] << 16)) < 65520.f);
    bad += !(fabsf(__uint_as_float(v[j] & 0xFFFF0000u)) < 65520.f);
  }
  if (bad && n_overflow) atomicAdd(n_overflow, bad);
}

}  // namespace

int plan_gemm(GemmArgs& g, int dtype) {
  if (dtype == 0) {
    g.kind = GEMM_F32;
    const int tiles = ((g.N + 63) / 64) * ((g.M + 15) / 16);
    int S = 1;
    while (tiles * S < 256 && (g.K % (2 * S * 32)) == 0 && g.K / (2 * S) >= 64) S *= 2;
    g.S = S;
    g.kc = g.K / S;
    return S;
  }
  if (g.M <= 64) {
    const int MT = g.M <= 16 ? 1 : (g.M <= 32 ? 2 : 4);
    g.kind = MT == 1 ? GEMM_SKINNY1 : (MT == 2 ? GEMM_SKINNY2 : GEMM_SKINNY4);
    const int ntiles = (g.N + SK_NT - 1) / SK_NT;
    const int kmax = 2048 / MT;  // staged A slice <= 64 KB of LDS
    // 1024-wide slices for the large matrices (fewer partial sums to reduce), else 512
    int kc = (long long)g.N * g.K >= (48ll << 20) ? 1024 : 512;
    if (kc > kmax) kc = kmax;
    // a split must not straddle two A segments: kc | ka_w (ka_w = K for one segment)
    while (kc > 256 && (g.K % kc || g.ka_w % kc)) kc >>= 1;
    if (kc < 256 || g.K % kc || g.ka_w % kc) kc = (g.K % 256 == 0 && g.ka_w % 256 == 0) ? 256 : 0;
    g.kc = kc;
    g.S = kc ? g.K / kc : 0;
    if (g.S) {
      // ~SK_GRID workgroups: wps per split, each with tpw tiles (the last ones one fewer)
      int wps = SK_GRID / g.S;
      if (wps < 1) wps = 1;
      if (wps > ntiles) wps = ntiles;
      const int tpw = (ntiles + wps - 1) / wps;
      g.wps = (ntiles + tpw - 1) / tpw;
      g.grid = g.S * g.wps;
    }
    return g.S;
  }
  g.kind = GEMM_MFMA;
  const int KT = g.K / 32;
  // 128 x 128 tiles for at most 128 rows, where a 256-row tile would be half padding
  g.tile = g.M <= MF_SMALL_ROWS ? 128 : 256;
  const int tiles = ((g.N + g.tile - 1) / g.tile) * ((g.M + g.tile - 1) / g.tile);
  const int slots = 256;
  // split K so that tiles x S fills up to one round of resident workgroups,
  // keeping at least 16 k steps per split
  int S = tiles >= slots ? 1 : slots / tiles;
  if (S > 8) S = 8;
  if (S > KT / 16) S = KT / 16 > 0 ? KT / 16 : 1;
  const int ksteps = (KT + S - 1) / S;
  g.kc = ksteps * 32;
  g.S = (KT + ksteps - 1) / ksteps;
  return g.S;
}

bool plan_swiglu(GemmArgs& g) {
  const int I = g.N / 2;
  if (g.kind != GEMM_MFMA || g.tile != 256 || g.S != 1 || g.n_wseg != 2 || g.n_off[1] != I ||
      I % 128)
    return false;
  if (I % 192 == 0) {
    // The tiles run one workgroup per CU: a launch takes as many rounds as it has
    // tiles per 256 CUs, and a 128 x 384 tile costs 7/8 of a 256 x 256 one (its LDS
    // traffic per k step, which bounds both: 112 KB against 128 KB).  At 512 rows
    // and I = 12288 that is 256 tiles in one round against 192 tiles (a quarter of
    // the CUs idle) in one round of the longer tile.
    auto rounds = [&](int tm, int tn) {
      const long long t = (long long)((g.M + tm - 1) / tm) * (g.N / tn);
      return (t + 255) / 256;
    };
    if (rounds(128, 384) * 7 < rounds(256, 256) * 8) g.tile = 384;
  }
  return true;
}

hipError_t launch_gemm(const GemmArgs& g, int dtype, hipStream_t st, LaunchEvents ev) {
  (void)dtype;
  switch (g.kind) {
    case GEMM_F32: {
      dim3 grid((g.N + 63) / 64, (g.M + 15) / 16, g.S);
      DF_LAUNCH(ev.start, ev.stop, gemm_f32, grid, 256, 0, st, g);
      break;
    }
    case GEMM_SKINNY1:
    case GEMM_SKINNY2:
    case GEMM_SKINNY4: {
      if (g.S <= 0 || g.grid <= 0 || g.K % 32 || g.N % 16 || g.ka_w % g.kc) return hipErrorInvalidValue;
      if (g.nss && g.nss_chunks > 512) return hipErrorInvalidValue;  // row statistics: 16 threads x 32
      const int MT = g.kind == GEMM_SKINNY1 ? 1 : (g.kind == GEMM_SKINNY2 ? 2 : 4);
      if (g.kc * MT > 2048) return hipErrorInvalidValue;  // LDS
      const size_t lds = (size_t)(g.kc / 32) * MT * 64 * 16;
#define SK_LAUNCH(mt)                                                                         \
  if (g.a_f32) DF_LAUNCH(ev.start, ev.stop, (gemm_skinny<mt, true>), g.grid, SK_THREADS, lds, st, g); \
  else DF_LAUNCH(ev.start, ev.stop, (gemm_skinny<mt, false>), g.grid, SK_THREADS, lds, st, g);
      if (MT == 1) { SK_LAUNCH(1) }
      else if (MT == 2) { SK_LAUNCH(2) }
      else { SK_LAUNCH(4) }
#undef SK_LAUNCH
      break;
    }
    case GEMM_MFMA: {
      if (g.K % 32 || g.N % 16 || !g.apack || g.S <= 0 ||
          (g.tile != 256 && g.tile != 128 && g.tile != 384))
        return hipErrorInvalidValue;
      // 384: 128 x 384 tiles, for the SwiGLU epilogue only
      if (g.tile == 384 && !g.swiglu_out) return hipErrorInvalidValue;
      if (g.swiglu_out && (g.tile == 128 || g.S != 1 || g.n_wseg != 2 || g.N % g.tile ||
                           g.n_off[1] != g.N / 2))
        return hipErrorInvalidValue;
      const int TM = g.tile == 384 ? 128 : g.tile, TN = g.tile;
      const void* kern = g.tile == 256   ? (const void*)gemm_mfma<256, 256>
                         : g.tile == 384 ? (const void*)gemm_mfma<128, 384>
                                         : (const void*)gemm_mfma<128, 128>;
      const int lds = g.tile == 256   ? MfTile<256, 256>::LDS
                      : g.tile == 384 ? MfTile<128, 384>::LDS
                                      : MfTile<128, 128>::LDS;
      const hipError_t ae = set_lds_limit(kern, lds);
      if (ae != hipSuccess) return ae;
      const int mpad = (g.M + MF_M - 1) / MF_M * MF_M;  // packed A rows (whole 256-row tiles)
      dim3 pgrid(mpad / 16, (g.K / 32 + 7) / 8);
      hipEvent_t none = nullptr, gstart = ev.start;
      if (!g.a_packed) {
        if (g.a_f32) DF_LAUNCH(ev.start, none, pack_rows_k<true>, pgrid, 256, 0, st, g);
        else DF_LAUNCH(ev.start, none, pack_rows_k<false>, pgrid, 256, 0, st, g);
        gstart = none;
      }
      const int n_mt = (g.M + TM - 1) / TM, n_nt = (g.N + TN - 1) / TN;
      const int per = xcd_per(n_mt * n_nt * g.S);
      if (g.tile == 256)
        DF_LAUNCH(gstart, ev.stop, (gemm_mfma<256, 256>), 8 * per, MF_WAVES * 64, lds, st, g, n_mt,
                  n_nt, per);
      else if (g.tile == 384)
        DF_LAUNCH(gstart, ev.stop, (gemm_mfma<128, 384>), 8 * per, MF_WAVES * 64, lds, st, g, n_mt,
                  n_nt, per);
      else
        DF_LAUNCH(gstart, ev.stop, (gemm_mfma<128, 128>), 8 * per, MF_WAVES * 64, lds, st, g, n_mt,
                  n_nt, per);
      break;
    }
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// one-stream configuration by K
static bool rowk_long(int K) { return K > 4096; }
static int rowk_step(int K, bool gate_up) {
  if (gate_up) return 32 * RK_KW2 * 2 * RK_U2;
  return rowk_long(K) ? 32 * RK_KW_L * 2 * RK_U_L : 32 * RK_KW_S * 2 * RK_U_S;
}

bool rowk_fits(int M, int N, int K, bool gate_up) {
  return M >= 1 && M <= 16 && N % 16 == 0 && K % rowk_step(K, gate_up) == 0 && SS_COLS == 16;
}

static bool rowk_ss_ok(const float* ss, int nch, int kw) {
  return ss && nch % (16 * kw) == 0 && nch / (4 * kw) <= 4 * RK_SSV;
}

bool rowk_qkv_fits(int M, int K, int d) {
  return M >= 1 && M <= 16 && d % 32 == 0 && K % (32 * RK_KWQ * 2 * RK_UQ) == 0 &&
         K / 16 % (16 * RK_KWQ) == 0 && K / 16 / (4 * RK_KWQ) <= 4 * RK_SSV;
}

hipError_t launch_rowk_qkv(const void* A, const void* Wq, const void* Wk, const void* Wv, int M,
                           int K, int B, int Hq, int Hkv, int d, const float* ss_in, float eps,
                           const float* sc, const int32_t* len, const float* rope, float* q,
                           void* kc, void* vc, int max_ctx, hipStream_t st, LaunchEvents ev) {
  if (!rowk_qkv_fits(M, K, d) || !A || !Wq || !Wk || !Wv || !ss_in || !sc || !len || !rope ||
      !q || !kc || !vc || B < 1 || max_ctx % 32)
    return hipErrorInvalidValue;
  RowkArgs r{};
  r.A = (const f16_t*)A, r.W = (const f16_t*)Wq, r.W2 = (const f16_t*)Wk, r.Wv = (const f16_t*)Wv;
  r.M = M, r.N = (Hq + 2 * Hkv) * d, r.K = K;
  r.ss_in = ss_in, r.nch_in = K / 16, r.eps = eps, r.sc = (float*)sc;
  r.len = len, r.rope = rope, r.q = q, r.kc = (f16_t*)kc, r.vc = (f16_t*)vc;
  r.B = B, r.Hq = Hq, r.Hkv = Hkv, r.d = d, r.max_ctx = max_ctx;
  const int grid = (Hq + 2 * Hkv) * (d / 32);
  DF_LAUNCH(ev.start, ev.stop, (gemm_rowk<RK_QKV, RK_KWQ, RK_UQ>), grid, RK_KWQ * 64, 0, st, r);
  return hipGetLastError();
}

hipError_t launch_rowk_resid(const void* A, const void* W, int M, int N, int K, float* X,
                             float* ss_out, hipStream_t st, LaunchEvents ev) {
  if (!rowk_fits(M, N, K, false) || !A || !W || !X || !ss_out) return hipErrorInvalidValue;
  RowkArgs r{};
  r.A = (const f16_t*)A, r.W = (const f16_t*)W, r.M = M, r.N = N, r.K = K, r.X = X, r.ss_out = ss_out;
  if (rowk_long(K))
    DF_LAUNCH(ev.start, ev.stop, (gemm_rowk<RK_RESID, RK_KW_L, RK_U_L>), N / 16, RK_KW_L * 64, 0,
              st, r);
  else
    DF_LAUNCH(ev.start, ev.stop, (gemm_rowk<RK_RESID, RK_KW_S, RK_U_S>), N / 16, RK_KW_S * 64, 0,
              st, r);
  return hipGetLastError();
}

hipError_t launch_rowk_resid_y(const void* A, const void* W, int M, int N, int K, float* X,
                               float* ss_out, const float* ss_in, const void* gain, float eps,
                               float* sc, void* y, hipStream_t st, LaunchEvents ev) {
  if (!rowk_fits(M, N, K, false) || !A || !W || !X || !ss_out ||
      !rowk_ss_ok(ss_in, N / 16, rowk_long(K) ? RK_KW_L : RK_KW_S) ||
      !gain || !sc || !y || ss_in == ss_out)
    return hipErrorInvalidValue;
  RowkArgs r{};
  r.A = (const f16_t*)A, r.W = (const f16_t*)W, r.M = M, r.N = N, r.K = K, r.X = X, r.ss_out = ss_out;
  r.ss_in = ss_in, r.nch_in = N / 16, r.gain = (const bf16_t*)gain, r.eps = eps, r.sc = sc;
  r.out16 = (f16_t*)y;
  if (rowk_long(K))
    DF_LAUNCH(ev.start, ev.stop, (gemm_rowk<RK_RESID_Y, RK_KW_L, RK_U_L>), N / 16, RK_KW_L * 64,
              0, st, r);
  else
    DF_LAUNCH(ev.start, ev.stop, (gemm_rowk<RK_RESID_Y, RK_KW_S, RK_U_S>), N / 16, RK_KW_S * 64,
              0, st, r);
  return hipGetLastError();
}

hipError_t launch_rowk_swiglu(const void* A, const void* Wg, const void* Wu, int M, int I, int K,
                              const float* ss_in, float eps, const float* sc, void* out,
                              hipStream_t st, LaunchEvents ev) {
  if (!rowk_fits(M, I, K, true) || I % 32 || !A || !Wg || !Wu || !rowk_ss_ok(ss_in, K / 16, RK_KW2) ||
      !sc || !out)
    return hipErrorInvalidValue;
  RowkArgs r{};
  r.A = (const f16_t*)A, r.W = (const f16_t*)Wg, r.W2 = (const f16_t*)Wu, r.M = M, r.N = I, r.K = K;
  r.ss_in = ss_in, r.nch_in = K / 16, r.eps = eps, r.sc = (float*)sc, r.out16 = (f16_t*)out;
  DF_LAUNCH(ev.start, ev.stop, (gemm_rowk<RK_SWIGLU, RK_KW2, RK_U2>), I / 16, RK_KW2 * 64, 0, st,
            r);
  return hipGetLastError();
}

size_t gemm_apack_bytes(const GemmArgs& g) {
  if (g.kind != GEMM_MFMA) return 0;
  return (size_t)((g.M + MF_M - 1) / MF_M * MF_M) * g.K * 2;
}

hipError_t launch_pack_weight(const void* src, int N, int K, void* dst, int32_t* n_overflow,
                              hipStream_t st) {
  if (N % 16 || K % 32) return hipErrorInvalidValue;
  const long long npiece = (long long)N * K / 8;
  if (npiece == 0) return hipSuccess;
  pack_weight_k<<<(unsigned)((npiece + 255) / 256), 256, 0, st>>>((const bf16_t*)src, N, K,
                                                                   (f16_t*)dst, n_overflow);
  return hipGetLastError();
}
