// Projection GEMMs of the drafter: out[s][m][n] = sum_{k in split s} A[m,k] * W[n,k].
//
// Three kernels, chosen by shape:
//  * skinny (bf16, M <= 64): weight streaming.  Each workgroup owns 64 output
//    columns (16 per wave) and one K split; the activation slice A[:, split]
//    is staged once in LDS, already in MFMA fragment order, and every wave
//    streams its 16 weight rows with 16-byte loads, prefetching U k-steps
//    ahead, into v_mfma_f32_16x16x32_bf16.  At M = batch*16 the arithmetic
//    intensity is ~16 flop/B, far below the MFMA ridge, so the kernel is
//    HBM-bound; the matrix cores only keep the 16-row FMA work off the VALU.
//  * big (bf16, M > 64): 128x128x64 LDS tiles, double buffered, four waves of
//    64x64 built from v_mfma_f32_32x32x16_bf16.
//  * f32: a plain LDS-tiled FMA kernel for the fp32 storage type.
// Partial sums over K splits are reduced, in split order, by the consumer
// kernel, which also applies the epilogue (residual, norm, RoPE, SwiGLU).

#include "common.h"
#include "kernels.h"

namespace {

constexpr int SK_U = 8;        // k-steps (of 32) prefetched per wave
constexpr int SK_NT = 64;      // output columns per skinny workgroup

__device__ __forceinline__ const bf16_t* a_ptr(const GemmArgs& g, int row, int k) {
  const int seg = k / g.ka_w;
  return (const bf16_t*)g.a[seg] + (long long)row * g.lda + (k - seg * g.ka_w);
}

__device__ __forceinline__ const bf16_t* w_row_ptr(const GemmArgs& g, int n, bool& ok) {
  ok = n < g.N;
  if (!ok) return (const bf16_t*)g.w[0];
  int j = 0;
  while (j + 1 < g.n_wseg && n >= g.n_off[j + 1]) ++j;
  return (const bf16_t*)g.w[j] + (long long)(n - g.n_off[j]) * g.ldw;
}

template <int MT>
__global__ __launch_bounds__(256) void gemm_skinny_bf16(GemmArgs g) {
  extern __shared__ bf16x8 sA[];  // [(t * MT + mt) * 64 + lane]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int s = blockIdx.y;
  const int k0 = s * g.kc;
  const int T = g.kc / 32;

  const int n = blockIdx.x * SK_NT + wave * 16 + (lane & 15);
  bool nok;
  const bf16_t* wp = w_row_ptr(g, n, nok) + k0 + (lane >> 4) * 8;

  bf16x8 cur[SK_U], nxt[SK_U];
#pragma unroll
  for (int u = 0; u < SK_U; ++u) cur[u] = *(const bf16x8*)(wp + u * 32);

  // stage A[:, k0:k0+kc] in fragment order: slot (t, mt, l) = A[mt*16 + l%16][k0 + 32t + 8(l/16) ..+8]
  const int nslots = T * MT * 64;
  for (int p = threadIdx.x; p < nslots; p += 256) {
    const int l = p & 63;
    const int tm = p >> 6;
    const int mt = tm % MT, t = tm / MT;
    const int row = mt * 16 + (l & 15);
    bf16x8 v = {};
    if (row < g.M) v = *(const bf16x8*)a_ptr(g, row, k0 + t * 32 + (l >> 4) * 8);
    sA[p] = v;
  }
  __syncthreads();

  floatx4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int t0 = 0; t0 < T; t0 += SK_U) {
    if (t0 + SK_U < T) {
#pragma unroll
      for (int u = 0; u < SK_U; ++u) nxt[u] = *(const bf16x8*)(wp + (t0 + SK_U + u) * 32);
    }
#pragma unroll
    for (int u = 0; u < SK_U; ++u) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8 a = sA[((t0 + u) * MT + mt) * 64 + lane];
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, cur[u], acc[mt], 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < SK_U; ++u) cur[u] = nxt[u];
  }

  if (!nok) return;
  float* out = g.out + (long long)s * g.M * g.N;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mt * 16 + (lane >> 4) * 4 + i;
      if (m < g.M) out[(long long)m * g.N + n] = acc[mt][i];
    }
  }
}

// ---- big tiles ------------------------------------------------------------------
constexpr int BG_M = 128, BG_N = 128, BG_K = 64, BG_LD = BG_K + 8;  // LDS row pitch (elements)

__global__ __launch_bounds__(256) void gemm_big_bf16(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][BG_M * BG_LD];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][BG_N * BG_LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.y * BG_M, n0 = blockIdx.x * BG_N;
  const int s = blockIdx.z;
  const int kbeg = s * g.kc, nk = g.kc / BG_K;

  // each thread moves 4 A pieces and 4 B pieces (16 bytes each) per k-tile
  int prow[4], pcol[4];
  const bf16_t* brow[4];
  bool aok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = tid + 256 * i;
    prow[i] = p >> 3;
    pcol[i] = (p & 7) * 8;
    aok[i] = (m0 + prow[i]) < g.M;
    bool ok;
    brow[i] = w_row_ptr(g, n0 + prow[i], ok);
  }
  u32x4 ra[4], rb[4];
  auto gload = [&](int kt) {
    const int k = kbeg + kt * BG_K;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = aok[i] ? *(const u32x4*)a_ptr(g, m0 + prow[i], k + pcol[i]) : u32x4{0, 0, 0, 0};
      rb[i] = *(const u32x4*)(brow[i] + k + pcol[i]);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *(u32x4*)&sA[buf][prow[i] * BG_LD + pcol[i]] = ra[i];
      *(u32x4*)&sB[buf][prow[i] * BG_LD + pcol[i]] = rb[i];
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
    for (int kk = 0; kk < BG_K / 16; ++kk) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *(const bf16x8*)&sA[buf][(wm * 64 + i * 32 + (lane & 31)) * BG_LD + kk * 16 + (lane >> 5) * 8];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = *(const bf16x8*)&sB[buf][(wn * 64 + j * 32 + (lane & 31)) * BG_LD + kk * 16 + (lane >> 5) * 8];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
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
  const int tid = threadIdx.x;
  const int m0 = blockIdx.y * 16, n0 = blockIdx.x * 64;
  const int s = blockIdx.z;
  const int col = tid & 63, rg = tid >> 6;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const int kbeg = s * g.kc, kend = kbeg + g.kc;
  // weight row pointers for the 8 W-tile loads of this thread
  for (int k0 = kbeg; k0 < kend; k0 += 32) {
    for (int p = tid; p < 16 * 32; p += 256) {
      const int r = p >> 5, c = p & 31;
      const int m = m0 + r, k = k0 + c;
      float v = 0.f;
      if (m < g.M) {
        const int seg = k / g.ka_w;
        v = ((const float*)g.a[seg])[(long long)m * g.lda + (k - seg * g.ka_w)];
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

}  // namespace

int plan_gemm(GemmArgs& g, int dtype) {
  if (dtype == 0) {
    g.kind = GEMM_F32;
    // enough workgroups for small problems: split K in 64-wide pieces
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
    const int kmax = 1024 / MT;
    int kc = 0;
    for (int c = kmax; c >= 256; c >>= 1) {
      if (g.K % c) continue;
      kc = c;
      if ((long long)ntiles * (g.K / c) >= 512) break;
    }
    g.kc = kc;
    g.S = kc ? g.K / kc : 0;
    return g.S;
  }
  g.kind = GEMM_BIG;
  const int tiles = ((g.N + BG_N - 1) / BG_N) * ((g.M + BG_M - 1) / BG_M);
  int S = 1;
  while (tiles * S < 256 && S < 8 && g.K % (2 * S * BG_K) == 0) S *= 2;
  g.S = S;
  g.kc = g.K / S;
  return S;
}

hipError_t launch_gemm(const GemmArgs& g, int dtype, hipStream_t st) {
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
      dim3 grid((g.N + SK_NT - 1) / SK_NT, g.S);
      const size_t lds = (size_t)(g.kc / 32) * MT * 64 * 16;
      if (MT == 1) gemm_skinny_bf16<1><<<grid, 256, lds, st>>>(g);
      else if (MT == 2) gemm_skinny_bf16<2><<<grid, 256, lds, st>>>(g);
      else gemm_skinny_bf16<4><<<grid, 256, lds, st>>>(g);
      break;
    }
    case GEMM_BIG: {
      dim3 grid((g.N + BG_N - 1) / BG_N, (g.M + BG_M - 1) / BG_M, g.S);
      gemm_big_bf16<<<grid, 256, 0, st>>>(g);
      break;
    }
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
