// Projection GEMMs of the drafter: out[s][m][n] = sum_{k in split s} A[m,k] * W[n,k].
//
// W is bf16 (or fp32 for the fp32 storage type) and streams from HBM once.
// A is either bf16 (the target features, exact) or an fp32 activation; fp32
// activations enter the bf16 MFMA as a hi+lo pair (x = hi + lo, two MFMAs),
// so the product carries ~16 mantissa bits of A and the exact bf16 weight.
//
// Three kernels, chosen by shape:
//  * skinny (bf16 W, M <= 64): weight streaming.  Each workgroup owns 64
//    output columns (16 per wave) and one K split; the activation slice
//    A[:, split] is staged once in LDS, already split and in MFMA fragment
//    order, and every wave streams its 16 weight rows with 16-byte loads,
//    prefetching U k-steps ahead, into v_mfma_f32_16x16x32_bf16.  At
//    M = batch*16 the arithmetic intensity is ~16-32 flop/B, far below the
//    MFMA ridge: the kernel is HBM-bound and the matrix cores only keep the
//    FMA work off the VALU.
//  * big (bf16 W, M > 64): 128x128 LDS tiles, double buffered, four waves of
//    64x64 built from v_mfma_f32_32x32x16_bf16.
//  * f32: a plain LDS-tiled FMA kernel for the fp32 storage type.
// Partial sums over K splits are reduced, in split order, by the consumer
// kernel, which also applies the epilogue (residual, norm, RoPE, SwiGLU).

#include "common.h"
#include "kernels.h"

namespace {

constexpr int SK_U = 8;            // k-steps (of 32) per prefetch buffer
constexpr int SK_THREADS = 512;    // 8 waves
constexpr int SK_NT = 128;         // output columns per tile (16 per wave)

template <typename TA>
__device__ __forceinline__ const TA* a_ptr(const GemmArgs& g, int row, int k) {
  const int seg = k / g.ka_w;
  return (const TA*)g.a[seg] + (long long)row * g.lda + (k - seg * g.ka_w);
}

__device__ __forceinline__ const bf16_t* w_row_ptr(const GemmArgs& g, int n, bool& ok) {
  ok = n < g.N;
  if (!ok) return (const bf16_t*)g.w[0];
  if (g.il) {  // 128-column tiles: 64 rows of segment 0, then the same 64 rows of segment 1
    const int t = n >> 7, c = n & 127;
    return (const bf16_t*)g.w[c >> 6] + (long long)(t * 64 + (c & 63)) * g.ldw;
  }
  int j = 0;
  while (j + 1 < g.n_wseg && n >= g.n_off[j + 1]) ++j;
  return (const bf16_t*)g.w[j] + (long long)(n - g.n_off[j]) * g.ldw;
}

// 1 / RMS of A row `row` from its partial sums of squares (norm folded into staging).
__device__ __forceinline__ float row_rs(const GemmArgs& g, int row) {
  float t = 0.f;
  for (int c = 0; c < g.nss_chunks; ++c) t += g.nss[(long long)row * g.nss_chunks + c];
  return rsqrtf(t / g.K + g.neps);
}

// A fragment (8 consecutive k of one row) as bf16 hi (+ lo when SPLIT); fp32 A rows
// are scaled by rs * gain[k] first when a norm is folded in.
template <bool SPLIT>
__device__ __forceinline__ void load_a8(const GemmArgs& g, int row, int k, float rs, bf16x8& hi,
                                        bf16x8& lo) {
  if (SPLIT) {
    const float* p = a_ptr<float>(g, row, k);
    floatx4 a = *(const floatx4*)p, b = *(const floatx4*)(p + 4);
    if (g.nss) {
      const bf16x8 gw = *(const bf16x8*)((const bf16_t*)g.ngain + k);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a[j] *= rs * (float)gw[j];
        b[j] *= rs * (float)gw[4 + j];
      }
    }
    split8v(a, b, hi, lo);
  } else {
    hi = *(const bf16x8*)a_ptr<bf16_t>(g, row, k);
  }
}

// ---- fused epilogue of one 128-column tile (skinny GEMMs) ---------------------------
__device__ void skinny_epilogue(const GemmArgs& g, int tile) {
  const EpiArgs& e = g.e;
  const int tid = threadIdx.x;
  const int n0 = tile * SK_NT;
  const int M = g.M, N = g.N, S = g.S;
  const long long sstride = (long long)M * N;
  auto sumP = [&](int m, int n) {
    const float* p = g.out + (long long)m * N + n;
    float v = 0.f;
    for (int s = 0; s < S; ++s) v += p[s * sstride];
    return v;
  };
  auto sumP4 = [&](int m, int n) {  // 4 consecutive columns, n % 4 == 0
    const floatx4* p = (const floatx4*)(g.out + (long long)m * N + n);
    floatx4 v = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < S; ++s) v += p[s * sstride / 4];
    return v;
  };
  const int part = tid & 31;  // 32 threads per row, 16 rows per pass
  if (e.kind == EPI_ROWS || e.kind == EPI_RESID) {
    const int nch = (N + SS_COLS - 1) / SS_COLS;
    for (int m = tid >> 5; m < M; m += SK_THREADS / 32) {
      float sq = 0.f;
      const int n = n0 + part * 4;
      if (n < N) {
        floatx4 v = sumP4(m, n);
        floatx4* xp = (floatx4*)(e.x + (long long)m * N + n);
        if (e.kind == EPI_RESID) v += *xp;
        *xp = v;
        sq = v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
      }
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) sq += __shfl_xor(sq, o, 64);
      if (part == 0) e.ss[(long long)m * nch + tile] = sq;
    }
  } else if (e.kind == EPI_SWIGLU) {
    const int I = N / 2;
    for (int m = tid >> 5; m < M; m += SK_THREADS / 32) {
      if (part < 16) {  // 16 threads x 4 columns = the tile's 64 gate | 64 up pairs
        const int c = part * 4;
        if (tile * 64 + c < I) {
          const floatx4 gt = sumP4(m, n0 + c), up = sumP4(m, n0 + 64 + c);
          floatx4 r;
#pragma unroll
          for (int j = 0; j < 4; ++j) r[j] = gt[j] / (1.f + __expf(-gt[j])) * up[j];
          *(floatx4*)(e.act + (long long)m * I + tile * 64 + c) = r;
        }
      }
    }
  } else if (e.kind == EPI_QKV || e.kind == EPI_INJECT) {
    const int d = e.d, half = d >> 1;
    const int KVD = e.Hkv * d;
    for (int m = tid >> 5; m < M; m += SK_THREADS / 32) {
      int b, pos;
      if (e.kind == EPI_QKV) {
        b = m / e.B;
        pos = e.len[b] + m % e.B;
      } else {
        b = e.seq[m];
        pos = e.pos[m];
        if (b < 0) continue;
      }
      const bool wr = pos < e.max_ctx;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int pslot = part + 32 * j;               // 64 column pairs per tile
        const int ht = pslot / half, i = pslot % half;
        const int c1 = n0 + ht * d + i, c2 = c1 + half;
        if (c2 >= N) continue;
        const float x1 = sumP(m, c1), x2 = sumP(m, c2);
        if (e.kind == EPI_QKV) {
          const int hh = c1 / d;                      // head in [q | k | v]
          if (hh < e.Hq + e.Hkv) {
            const float cs = e.rope[((long long)m * half + i) * 2];
            const float sn = e.rope[((long long)m * half + i) * 2 + 1];
            const float y1 = x1 * cs - x2 * sn, y2 = x2 * cs + x1 * sn;
            if (hh < e.Hq) {
              float* qo = e.q + (long long)m * e.Hq * d + hh * d;
              qo[i] = y1;
              qo[i + half] = y2;
            } else if (wr) {
              float* ko = e.kc + (((long long)b * e.Hkv + (hh - e.Hq)) * e.max_ctx + pos) * d;
              ko[i] = y1;
              ko[i + half] = y2;
            }
          } else if (wr) {
            const int kh = hh - e.Hq - e.Hkv;
            float* vo = e.vc + ((long long)b * e.Hkv + kh) * d * (long long)e.max_ctx + pos;
            vo[(long long)i * e.max_ctx] = x1;
            vo[(long long)(i + half) * e.max_ctx] = x2;
          }
        } else if (wr) {
          const int l = c1 / (2 * KVD), jj = c1 % (2 * KVD);
          const int kh = (jj % KVD) / d;
          if (jj < KVD) {
            const double inv = exp(-(2.0 * i / d) * log((double)e.theta));
            double sd, cd;
            sincos((double)pos * inv, &sd, &cd);
            const float cs = (float)cd, sn = (float)sd;
            float* ko = (float*)e.cp.k[l] + (((long long)b * e.Hkv + kh) * e.max_ctx + pos) * d;
            ko[i] = x1 * cs - x2 * sn;
            ko[i + half] = x2 * cs + x1 * sn;
          } else {
            float* vo = (float*)e.cp.v[l] + ((long long)b * e.Hkv + kh) * d * (long long)e.max_ctx + pos;
            vo[(long long)i * e.max_ctx] = x1;
            vo[(long long)(i + half) * e.max_ctx] = x2;
          }
        }
      }
    }
  }
}

// Skinny GEMM: workgroup (split s, index wi) stages A[:, split s] once, then
// streams the weights of tiles wi, wi + wps, ... .  With a fused epilogue, the
// last split to finish a tile reduces the S partials and applies it.
template <int MT, bool SPLIT>
__global__ __launch_bounds__(SK_THREADS) void gemm_skinny_bf16(GemmArgs g) {
  extern __shared__ bf16x8 sA[];  // hi: [(t * MT + mt) * 64 + lane], lo: + nslots
  __shared__ float srs[MT * 16];
  __shared__ int s_last;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int S = g.S;
  const int s = blockIdx.x % S;
  const int wi = blockIdx.x / S;
  const int k0 = s * g.kc;
  const int T = g.kc / 32;
  const int nslots = T * MT * 64;

  if (SPLIT && g.nss) {
    if (threadIdx.x < MT * 16 && (int)threadIdx.x < g.M) srs[threadIdx.x] = row_rs(g, threadIdx.x);
    __syncthreads();
  }
  // stage A[:, k0:k0+kc]: slot (t, mt, l) = A[mt*16 + l%16][k0 + 32t + 8(l/16) ..+8]
  for (int p = threadIdx.x; p < nslots; p += SK_THREADS) {
    const int l = p & 63;
    const int tm = p >> 6;
    const int mt = tm % MT, t = tm / MT;
    const int row = mt * 16 + (l & 15);
    bf16x8 hi = {}, lo = {};
    if (row < g.M)
      load_a8<SPLIT>(g, row, k0 + t * 32 + (l >> 4) * 8, (SPLIT && g.nss) ? srs[row] : 1.f, hi, lo);
    sA[p] = hi;
    if (SPLIT) sA[nslots + p] = lo;
  }
  __syncthreads();

  const int ntiles = (g.N + SK_NT - 1) / SK_NT;
  float* out = g.out + (long long)s * g.M * g.N;
  for (int tile = wi; tile < ntiles; tile += g.wps) {
    const int n = tile * SK_NT + wave * 16 + (lane & 15);
    bool nok;
    const bf16_t* wp = w_row_ptr(g, n, nok) + k0 + (lane >> 4) * 8;
    floatx4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
    stream_rows<SK_U, MT, SPLIT>(wp, T, sA, sA + nslots, lane, acc);
    const bool fused = g.e.kind != EPI_PARTIAL;
    if (nok) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = mt * 16 + (lane >> 4) * 4 + i;
          if (m < g.M) {
            if (fused) st_coherent(out + (long long)m * g.N + n, acc[mt][i]);
            else out[(long long)m * g.N + n] = acc[mt][i];
          }
        }
      }
    }
    if (fused && handoff_arrive(&g.e.cnt[tile], S - 1, &s_last)) {
      skinny_epilogue(g, tile);
      if (threadIdx.x == 0) g.e.cnt[tile] = 0;
    }
  }
}

// ---- big tiles ------------------------------------------------------------------
constexpr int BG_M = 128, BG_N = 128;

template <int BK, bool SPLIT>
__global__ __launch_bounds__(256) void gemm_big_bf16(GemmArgs g) {
  constexpr int LD = BK + 8;         // LDS row pitch (elements)
  constexpr int PP = BK / 16;        // 8-element pieces per thread per operand and k-tile
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][BG_M * LD];
  __shared__ __attribute__((aligned(16))) bf16_t sL[SPLIT ? 2 : 1][SPLIT ? BG_M * LD : 8];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][BG_N * LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.y * BG_M, n0 = blockIdx.x * BG_N;
  const int s = blockIdx.z;
  const int kbeg = s * g.kc, nk = g.kc / BK;

  int prow[PP], pcol[PP];
  const bf16_t* brow[PP];
  bool aok[PP];
  float prs[PP];
#pragma unroll
  for (int i = 0; i < PP; ++i) {
    const int p = tid + 256 * i;
    prow[i] = p / (BK / 8);
    pcol[i] = (p % (BK / 8)) * 8;
    aok[i] = (m0 + prow[i]) < g.M;
    prs[i] = (SPLIT && g.nss && aok[i]) ? row_rs(g, m0 + prow[i]) : 1.f;
    bool ok;
    brow[i] = w_row_ptr(g, n0 + prow[i], ok);
  }
  bf16x8 rah[PP], ral[PP], rb[PP];
  auto gload = [&](int kt) {
    const int k = kbeg + kt * BK;
#pragma unroll
    for (int i = 0; i < PP; ++i) {
      bf16x8 h = {}, l = {};
      if (aok[i]) load_a8<SPLIT>(g, m0 + prow[i], k + pcol[i], prs[i], h, l);
      rah[i] = h;
      ral[i] = l;
      rb[i] = *(const bf16x8*)(brow[i] + k + pcol[i]);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PP; ++i) {
      *(bf16x8*)&sA[buf][prow[i] * LD + pcol[i]] = rah[i];
      if (SPLIT) *(bf16x8*)&sL[buf][prow[i] * LD + pcol[i]] = ral[i];
      *(bf16x8*)&sB[buf][prow[i] * LD + pcol[i]] = rb[i];
    }
  };

  const int wm = wave >> 1, wn = wave & 1;
  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[2], al[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int off = (wm * 64 + i * 32 + (lane & 31)) * LD + kk * 16 + (lane >> 5) * 8;
        af[i] = *(const bf16x8*)&sA[buf][off];
        if (SPLIT) al[i] = *(const bf16x8*)&sL[buf][off];
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = *(const bf16x8*)&sB[buf][(wn * 64 + j * 32 + (lane & 31)) * LD + kk * 16 + (lane >> 5) * 8];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
          if (SPLIT)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  float* out = g.out + (long long)s * g.M * g.N;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + j * 32 + (lane & 31);
      if (n >= g.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (m < g.M) out[(long long)m * g.N + n] = acc[i][j][r];
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
    if (tid < 16 && m0 + tid < g.M) srs[tid] = row_rs(g, m0 + tid);
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
        v = *a_ptr<float>(g, m, k);
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

constexpr int big_bk(bool split) { return split ? 32 : 64; }

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
    const int kmax = (g.a_f32 ? 1024 : 2048) / MT;  // LDS: 64 KB for the staged A slice
    // largest K slice that still yields >= 256 (tile, split) items
    int kc = 0;
    for (int c = kmax; c >= 256; c >>= 1) {
      if (g.K % c) continue;
      kc = c;
      if ((long long)ntiles * (g.K / c) >= 256) break;
    }
    g.kc = kc;
    g.S = kc ? g.K / kc : 0;
    if (g.S) {
      const long long items = (long long)ntiles * g.S;
      const int tpw = items >= 1024 ? (int)(items / 512) : 1;  // tiles per workgroup
      g.wps = (ntiles + tpw - 1) / tpw;
    }
    return g.S;
  }
  g.kind = GEMM_BIG;
  const int bk = big_bk(g.a_f32);
  const int tiles = ((g.N + BG_N - 1) / BG_N) * ((g.M + BG_M - 1) / BG_M);
  int S = 1;
  while (tiles * S < 256 && S < 8 && g.K % (2 * S * bk) == 0) S *= 2;
  g.S = S;
  g.kc = g.K / S;
  return S;
}

hipError_t launch_gemm(const GemmArgs& g, int dtype, hipStream_t st) {
  (void)dtype;
  switch (g.kind) {
    case GEMM_F32: {
      dim3 grid((g.N + 63) / 64, (g.M + 15) / 16, g.S);
      gemm_f32<<<grid, 256, 0, st>>>(g);
      break;
    }
    case GEMM_SKINNY1:
    case GEMM_SKINNY2:
    case GEMM_SKINNY4: {
      const int MT = g.kind == GEMM_SKINNY1 ? 1 : (g.kind == GEMM_SKINNY2 ? 2 : 4);
      if (g.e.kind != EPI_PARTIAL && !g.e.cnt) return hipErrorInvalidValue;
      dim3 grid(g.S * g.wps);
      const size_t lds = (size_t)(g.kc / 32) * MT * 64 * 16 * (g.a_f32 ? 2 : 1);
#define SK_LAUNCH(mt)                                                                 \
  if (g.a_f32) gemm_skinny_bf16<mt, true><<<grid, SK_THREADS, lds, st>>>(g);         \
  else gemm_skinny_bf16<mt, false><<<grid, SK_THREADS, lds, st>>>(g);
      if (MT == 1) { SK_LAUNCH(1) }
      else if (MT == 2) { SK_LAUNCH(2) }
      else { SK_LAUNCH(4) }
#undef SK_LAUNCH
      break;
    }
    case GEMM_BIG: {
      dim3 grid((g.N + BG_N - 1) / BG_N, (g.M + BG_M - 1) / BG_M, g.S);
      if (g.a_f32) gemm_big_bf16<32, true><<<grid, 256, 0, st>>>(g);
      else gemm_big_bf16<64, false><<<grid, 256, 0, st>>>(g);
      break;
    }
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
