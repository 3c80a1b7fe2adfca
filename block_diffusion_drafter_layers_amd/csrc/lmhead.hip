// Shared lm_head with a fused greedy pick ("DFlash原理深度剖析", §二.3: the
// drafter reuses the target's output head; §二.1: the mask rows yield the
// candidate tokens).  Logits are reduced to (max, argmax) per row inside the
// kernel and never written, except by the debug variant that also stores them.
// Ties go to the lowest vocabulary id, here and in the cross-tile reduce.
//
// For the bf16 storage type the weight is fp16, fragment-packed (16 vocabulary
// rows x 32 k per 1 KB piece), and the normalised rows Z arrive as fp16.
// Rows <= 16 (batch 1): Z lives in LDS in MFMA fragment order (32*H bytes);
//   waves stride over 16-row vocabulary tiles and stream the 1.2 GB weight, one
//   contiguous 1 KB fragment per load instruction, into v_mfma_f32_16x16x32_f16;
//   each lane keeps a running best for its column slot, reduced across lanes
//   once at the end.
// Rows > 16: the rows arrive in the packed fragment layout too and 256x256 tiles
//   run the pipelined MFMA tile of the batched GEMM (mfma_tile.h) with an argmax
//   epilogue: per row, the best (value, id) over the tile's 256 ids.  A variant
//   with 128x128 tiles from row-major rows also stores every logit (parity hook).
// f32: one thread per vocabulary id, rows looped.

#include <math.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "mfma_tile.h"

namespace {

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// Folds the set (ov, oi, os) -- best score, its id, runner-up score -- into
// (v, i, s).  The runner-up of the union is the larger of both runner-ups and
// the best that lost (equal to the best on a tie).  fmaxf drops NaN.
__device__ __forceinline__ void top2_merge(float& v, int& i, float& s, float ov, int oi, float os) {
  if (better(ov, oi, v, i)) {
    s = fmaxf(fmaxf(s, os), v);
    v = ov;
    i = oi;
  } else {
    s = fmaxf(fmaxf(s, os), ov);
  }
}

// Gumbel noise of the ids v0 + 16 j (j = 0..3; bits 4 and 5 of v0 clear) for
// kernel row m: one Philox4x32-10 block at counter (v0, the row's position, its
// sequence, the offset) serves all four (see DraftSampler).
__device__ __forceinline__ void gumbel4(const DraftSampler& s, int m, int v0, float (&g)[4]) {
  const int b = m / s.rows_per_seq;
  const int pos = s.base[b] + m % s.rows_per_seq + 1;
  uint32_t c[4] = {(uint32_t)v0, (uint32_t)pos, (uint32_t)b, s.offset};
  philox4x32_10(c, s.k0, s.k1);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float u = (float)(2u * (c[j] >> 9) + 1u) * 0x1p-24f;  // exact: 2k + 1 < 2^24
    // u >= 2^-24 and -ln u >= 6e-8 are normal numbers, so the hardware base-2
    // logarithm (v_log_f32) scaled by ln 2 serves, without logf's denormal
    // scaling and two-part product
    constexpr float LN2 = 0.693147180559945f;
    const float nlu = -__builtin_amdgcn_logf(u) * LN2;  // -ln u > 0
    g[j] = -__builtin_amdgcn_logf(nlu) * LN2;
  }
}

// The score kernel row m gives id v: its logit, or with sampling logit / T plus
// the Gumbel noise of (v, the row's position, its sequence).  Rows at or past R
// (padding) never win.
template <bool SAMPLE>
__device__ __forceinline__ float draft_score(const DraftSampler& s, float logit, int m, int R, int v) {
  if (!SAMPLE) return logit;
  if (m >= R) return -INFINITY;
  float g[4];
  gumbel4(s, m, v & ~0x30, g);
  const int j = (v >> 4) & 3;  // selected, not indexed: g stays in registers
  return logit * s.inv_t + (j == 0 ? g[0] : j == 1 ? g[1] : j == 2 ? g[2] : g[3]);
}

constexpr int LH_U = 8;
constexpr int LH_WAVES = 8;

// PACKED: Z is one 16-row group of packed fp16 fragments (the layout sZ takes), R rows valid.
// SAMPLE: the Gumbel-max pick (a separate instantiation, so the greedy one keeps its registers).
template <bool PACKED, bool SAMPLE>
__global__ __launch_bounds__(LH_WAVES * 64) void lmhead_lds(int R, int V, int H, const f16_t* Z,
                                                            const f16_t* W, float* pval,
                                                            int32_t* pidx, float* logits,
                                                            DraftSampler smp) {
  extern __shared__ f16x8 sZ[];  // [t * 64 + lane]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int T = H / 32;
  // wave-major numbering: the waves that get one tile more than the others (ntile is
  // rarely a multiple of nw) are the low waves of every workgroup, so the last pass
  // spreads over every CU instead of filling the first ones and idling the rest
  const int gw = wave * gridDim.x + blockIdx.x;
  const int nw = gridDim.x * LH_WAVES;
  const int ntile = V / 16;
  // this wave's vocabulary tiles gw, gw + nw, ... (increasing ids)
  const int n_my = ntile > gw ? (ntile - gw + nw - 1) / nw : 0;
  auto tile_ptr = [&](int j) { return W + (long long)(gw + j * nw) * T * 512 + lane * 8; };
  f16x8 wa[LH_U];
  if (n_my > 0) load_w<LH_U>(wa, tile_ptr(0), 0);  // in flight while Z is staged
  for (int p = threadIdx.x; p < T * 64; p += blockDim.x) {
    const int l = p & 63, t = p >> 6;
    const int row = l & 15;
    f16x8 v = {};
    if (PACKED)
      v = ((const f16x8*)Z)[p];
    else if (row < R)
      v = *(const f16x8*)(Z + (long long)row * H + t * 32 + (l >> 4) * 8);
    sZ[p] = v;
  }
  __syncthreads();

  float best[4];
  int bidx[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    best[i] = -INFINITY;
    bidx[i] = 0x7fffffff;
  }
  if (n_my > 0)
    stream_tiles<LH_U, 1>(n_my, T, tile_ptr, sZ, lane, wa,
                                 [&](int j, const floatx4(&acc)[1]) {
#pragma unroll
                                   for (int i = 0; i < 4; ++i) {
                                     const int v = (gw + j * nw) * 16 + (lane & 15);
                                     const int row = (lane >> 4) * 4 + i;
                                     if (logits && row < R) logits[(long long)row * V + v] = acc[0][i];
                                     const float sv = draft_score<SAMPLE>(smp, acc[0][i], row, R, v);
                                     if (sv > best[i]) {  // tiles come in increasing id order
                                       best[i] = sv;
                                       bidx[i] = v;
                                     }
                                   }
                                 });
  // reduce over the 16 lanes of each lane group (same rows, different ids)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const float ov = __shfl_xor(best[i], o, 64);
      const int oi = __shfl_xor(bidx[i], o, 64);
      if (better(ov, oi, best[i], bidx[i])) {
        best[i] = ov;
        bidx[i] = oi;
      }
    }
  }
  if ((lane & 15) == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (lane >> 4) * 4 + i;
      if (row < R) {
        pval[(long long)gw * R + row] = best[i];
        pidx[(long long)gw * R + row] = bidx[i];
      }
    }
  }
}

// ---- many rows: 128 x 128 tiles with an argmax epilogue -----------------------------------
constexpr int LB_M = 128, LB_N = 128, LB_K = 64, LB_LD = LB_K + 8;

// pval2 (nullable): the runner-up score of each row over the tile's ids as well.
template <bool SAMPLE>
__global__ __launch_bounds__(256) void lmhead_tiled(int R, int V, int H, const f16_t* Z,
                                                    const f16_t* W, float* pval, int32_t* pidx,
                                                    float* pval2, float* logits, DraftSampler smp) {
  __shared__ __attribute__((aligned(16))) f16_t sA[2][LB_M * LB_LD];
  __shared__ __attribute__((aligned(16))) f16_t sB[2][LB_N * LB_LD];
  __shared__ float rv[2][LB_M];
  __shared__ int ri[2][LB_M];
  __shared__ float rs[2][LB_M];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.x * LB_M, n0 = blockIdx.y * LB_N;
  const int nk = H / LB_K;
  // A pieces: row p / 8, 8 columns at (p % 8) * 8.  B pieces: packed fragment
  // q = p / 64 of the tile (16-row group q % 8, k-step q / 8), lane slot p % 64.
  int prow[4], pcol[4], qrow[4], qcol[4];
  bool aok[4], bok[4];
  const f16_t* bsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = tid + 256 * i;
    prow[i] = p >> 3;
    pcol[i] = (p & 7) * 8;
    aok[i] = m0 + prow[i] < R;
    const int q = p >> 6, l = p & 63;
    qrow[i] = 16 * (q & 7) + (l & 15);
    qcol[i] = 32 * (q >> 3) + 8 * (l >> 4);
    const int grp = (n0 >> 4) + (q & 7);
    bok[i] = grp * 16 < V;
    bsrc[i] = W + ((long long)(bok[i] ? grp : 0) * (H / 32) + (q >> 3)) * 512 + l * 8;
  }
  u32x4 ra[4], rb[4];
  auto gload = [&](int kt) {
    const int k = kt * LB_K;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = aok[i] ? *(const u32x4*)(Z + (long long)(m0 + prow[i]) * H + k + pcol[i]) : u32x4{0, 0, 0, 0};
      rb[i] = bok[i] ? *(const u32x4*)(bsrc[i] + (long long)kt * (LB_K / 32) * 512) : u32x4{0, 0, 0, 0};
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *(u32x4*)&sA[buf][prow[i] * LB_LD + pcol[i]] = ra[i];
      *(u32x4*)&sB[buf][qrow[i] * LB_LD + qcol[i]] = rb[i];
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
    for (int kk = 0; kk < LB_K / 16; ++kk) {
      f16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *(const f16x8*)&sA[buf][(wm * 64 + i * 32 + (lane & 31)) * LB_LD + kk * 16 + (lane >> 5) * 8];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = *(const f16x8*)&sB[buf][(wn * 64 + j * 32 + (lane & 31)) * LB_LD + kk * 16 + (lane >> 5) * 8];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }
  // epilogue: per row, best over this wave's 64 columns, then over the two column waves;
  // the two row blocks are separate calls (i a constant in each), not an unrolled loop,
  // which the compiler declines for the sampling instantiation's size
  auto row_block = [&](auto ic) {
    constexpr int i = decltype(ic)::value;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ml = wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      float bv = -INFINITY, bs = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n0 + wn * 64 + j * 32 + (lane & 31);
        const float v = acc[i][j][r];
        if (n < V) {
          if (logits && m0 + ml < R) logits[(long long)(m0 + ml) * V + n] = v;
          const float sv = draft_score<SAMPLE>(smp, v, m0 + ml, R, n);
          top2_merge(bv, bi, bs, sv, n, -INFINITY);
        }
      }
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        const float os = __shfl_xor(bs, o, 64);
        top2_merge(bv, bi, bs, ov, oi, os);
      }
      if ((lane & 31) == 0) {
        rv[wn][ml] = bv;
        ri[wn][ml] = bi;
        rs[wn][ml] = bs;
      }
    }
  };
  row_block(std::integral_constant<int, 0>{});
  row_block(std::integral_constant<int, 1>{});
  __syncthreads();
  if (tid < LB_M) {
    float bv = rv[0][tid], bs = rs[0][tid];
    int bi = ri[0][tid];
    top2_merge(bv, bi, bs, rv[1][tid], ri[1][tid], rs[1][tid]);
    if (m0 + tid < R) {
      pval[(long long)blockIdx.y * R + m0 + tid] = bv;
      pidx[(long long)blockIdx.y * R + m0 + tid] = bi;
      if (pval2) pval2[(long long)blockIdx.y * R + m0 + tid] = bs;
    }
  }
}

// ---- many rows, packed: TM x 256 MFMA tiles with an argmax epilogue ----------------------
// Zp: R rows padded to a multiple of 256, packed.  TM = 256, or 128 for at most 128
// rows (half the matrix-core work of a 256-row tile that is mostly padding).
template <bool SAMPLE, int TM>
__global__ __launch_bounds__(MF_WAVES * 64) void lmhead_mfma(int R, int V, int H, const f16_t* Zp,
                                                            const f16_t* W, float* pval,
                                                            int32_t* pidx, int n_mt, int per_xcd,
                                                            DraftSampler smp) {
  extern __shared__ f16x8 smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // row tiles fastest: the row tiles of one vocabulary tile share its weights in L2
  const int t = xcd_tile(per_xcd);
  const int n_nt = (V + MF_N - 1) / MF_N;
  if (t >= n_mt * n_nt) return;
  const int mt = t % n_mt, nt = t / n_mt;
  const int KT = H / 32;
  using TL = MfTile<TM, MF_N>;
  constexpr int FPW = TL::FPW, FA = TL::FA, AG = TL::AG;
  const f16_t* src[FPW];
#pragma unroll
  for (int j = 0; j < FPW; ++j) {
    const int f = wave * FPW + j;
    int grp = nt * 16 + f - FA;
    if (grp * 16 >= V) grp = 0;  // past the vocabulary: any in-bounds group, masked below
    src[j] = (f < FA ? Zp + (long long)(mt * FA + f) * KT * 512 : W + (long long)grp * KT * 512) + lane * 8;
  }
  floatx4 acc[AG][4];
  mf_tile<TM, MF_N>(src, KT, smem, wave, lane, acc);
  const int wm = wave >> 2, wn = wave & 3;
  // best over this wave's 64 ids for each of its rows, then over the 16 lanes of a row group
  auto row_best = [&](int a, int r, float& v, int& id) {
    v = -INFINITY;
    id = 0x7fffffff;
    const int m = mt * TM + (AG * wm + a) * 16 + (lane >> 4) * 4 + r;
    // the lane's ids n0 + 16 b share one noise block (bits 4 and 5 of n0 are clear)
    const int n0 = nt * MF_N + 64 * wn + (lane & 15);
    float g[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (SAMPLE) {
      if (m < R) gumbel4(smp, m, n0, g);
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int n = n0 + 16 * b;
      if (n < V) {
        float sv = acc[a][b][r];
        if constexpr (SAMPLE) sv = m < R ? sv * smp.inv_t + g[b] : -INFINITY;
        if (better(sv, n, v, id)) {
          v = sv;
          id = n;
        }
      }
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const float ov = __shfl_xor(v, o, 64);
      const int oi = __shfl_xor(id, o, 64);
      if (better(ov, oi, v, id)) {
        v = ov;
        id = oi;
      }
    }
  };
  // across the four column waves, through LDS (the tile's stages are no longer read)
  float* rv = (float*)smem;                 // [4][TM]
  int* ri = (int*)((float*)smem + 4 * TM);  // [4][TM]
  if constexpr (SAMPLE) {
    // the noise needs registers: each row's best goes to LDS as soon as it is known
    __syncthreads();
#pragma unroll
    for (int a = 0; a < AG; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v;
        int id;
        row_best(a, r, v, id);
        if ((lane & 15) == 0) {
          const int row = (AG * wm + a) * 16 + (lane >> 4) * 4 + r;
          rv[wn * TM + row] = v;
          ri[wn * TM + row] = id;
        }
        // one row's noise at a time: interleaving rows would need more registers than there are
        __builtin_amdgcn_sched_barrier(0);
      }
  } else {
    float bv[AG][4];
    int bi[AG][4];
#pragma unroll
    for (int a = 0; a < AG; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) row_best(a, r, bv[a][r], bi[a][r]);
    __syncthreads();
    if ((lane & 15) == 0) {
#pragma unroll
      for (int a = 0; a < AG; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = (AG * wm + a) * 16 + (lane >> 4) * 4 + r;
          rv[wn * TM + row] = bv[a][r];
          ri[wn * TM + row] = bi[a][r];
        }
    }
  }
  __syncthreads();
  if (threadIdx.x < TM) {
    const int row = threadIdx.x;
    float v = rv[row];
    int id = ri[row];
#pragma unroll
    for (int w = 1; w < 4; ++w)
      if (better(rv[w * TM + row], ri[w * TM + row], v, id)) {
        v = rv[w * TM + row];
        id = ri[w * TM + row];
      }
    const int m = mt * TM + row;
    if (m < R) {
      pval[(long long)nt * R + m] = v;
      pidx[(long long)nt * R + m] = id;
    }
  }
}

// ---- f32 --------------------------------------------------------------------------------
template <bool SAMPLE>
__global__ __launch_bounds__(256) void lmhead_f32(int R, int V, int H, const float* Z,
                                                  const float* W, float* pval, int32_t* pidx,
                                                  float* pval2, float* logits, DraftSampler smp) {
  __shared__ float rv[4], rs[4];
  __shared__ int ri[4];
  const int v = blockIdx.x * 256 + threadIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int r = 0; r < R; ++r) {
    float s = -INFINITY;
    int id = 0x7fffffff;
    if (v < V) {
      const float* z = Z + (long long)r * H;
      const float* w = W + (long long)v * H;
      float a = 0.f;
      for (int k = 0; k < H; ++k) a = fmaf(z[k], w[k], a);
      if (logits) logits[(long long)r * V + v] = a;
      s = draft_score<SAMPLE>(smp, a, r, R, v);
      id = v;
    }
    float s2 = -INFINITY;  // runner-up: one id per lane, none yet
    for (int o = 1; o < 64; o <<= 1) {
      const float ov = __shfl_xor(s, o, 64);
      const int oi = __shfl_xor(id, o, 64);
      const float os = __shfl_xor(s2, o, 64);
      top2_merge(s, id, s2, ov, oi, os);
    }
    if (lane == 0) {
      rv[wave] = s;
      ri[wave] = id;
      rs[wave] = s2;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      float bv = rv[0], bs = rs[0];
      int bi = ri[0];
      for (int w = 1; w < 4; ++w) top2_merge(bv, bi, bs, rv[w], ri[w], rs[w]);
      pval[(long long)blockIdx.x * R + r] = bv;
      pidx[(long long)blockIdx.x * R + r] = bi;
      if (pval2) pval2[(long long)blockIdx.x * R + r] = bs;
    }
    __syncthreads();
  }
}

// Output row o; partials of row r = o, or (B > 0: the partials hold every row of
// whole B-row blocks) r = the row after the o % (B-1)-th of block o / (B-1).
// R = rows per partial tile.  pval2 (nullable): per-tile runner-up scores, then
// top2[o] = (best, runner-up) over all tiles.  A row whose best score is not
// finite (every score NaN, or an infinity) gets id 0 and raises
// DFLASH_ERR_NONFINITE.
__global__ __launch_bounds__(256) void argmax_reduce_k(int R, int ntiles, const float* pval,
                                                       const int32_t* pidx, const float* pval2,
                                                       int32_t* ids, int B, float* top2,
                                                       int32_t* err) {
  __shared__ float rv[4], rs[4];
  __shared__ int ri[4];
  const int o = blockIdx.x;
  const int r = B > 0 ? (o / (B - 1)) * B + o % (B - 1) + 1 : o;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float bv = -INFINITY, bs = -INFINITY;
  int bi = 0x7fffffff;
  for (int t0 = threadIdx.x; t0 < ntiles; t0 += 256 * 8) {  // 8 loads in flight per lane
    float v[8], v2[8];
    int id[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = min(t0 + 256 * j, ntiles - 1);
      v[j] = pval[(long long)t * R + r];
      id[j] = pidx[(long long)t * R + r];
      v2[j] = pval2 ? pval2[(long long)t * R + r] : -INFINITY;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (t0 + 256 * j < ntiles) top2_merge(bv, bi, bs, v[j], id[j], v2[j]);
  }
  for (int o = 1; o < 64; o <<= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    const float os = __shfl_xor(bs, o, 64);
    top2_merge(bv, bi, bs, ov, oi, os);
  }
  if (lane == 0) {
    rv[wave] = bv;
    ri[wave] = bi;
    rs[wave] = bs;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float v = rv[0], s2 = rs[0];
    int id = ri[0];
    for (int w = 1; w < 4; ++w) top2_merge(v, id, s2, rv[w], ri[w], rs[w]);
    if (!(fabsf(v) <= 3.402823466e38f)) {  // -inf: no score was a number; +inf or NaN
      set_err(err, 8);
      id = 0;
    }
    ids[o] = id;
    if (top2) {
      top2[2 * o] = v;
      top2[2 * o + 1] = s2;
    }
  }
}

constexpr int LH_GRID = 256;  // fixed grid: the partial count must not depend on the device

bool lds_variant(int R, int H) { return R <= 16 && H * 32 <= 160 * 1024; }

}  // namespace

bool lmhead_group_fits(int R, int H) { return R >= 1 && lds_variant(R, H) && H % 256 == 0; }

int lmhead_tiles(int dtype, int R, int V, int H, bool with_logits, bool top2) {
  if (dtype == 0) return (V + 255) / 256;
  if (top2) return (V + LB_N - 1) / LB_N;  // only the 128-wide tiles track the runner-up
  if (lds_variant(R, H)) return LH_GRID * LH_WAVES;
  // the packed matrix-core head (more than 16 rows, no logits) writes 256-wide tiles;
  // the 128-wide tiled head runs otherwise, also for at most 16 rows too wide for LDS
  return (!with_logits && R > 16) ? (V + MF_N - 1) / MF_N : (V + LB_N - 1) / LB_N;
}

// raises the dynamic-LDS limit of kernel k (once per kernel and device)
#define LH_ATTR(k, bytes)                                                                         \
  {                                                                                              \
    const hipError_t e = set_lds_limit((const void*)(k), (bytes));                               \
    if (e != hipSuccess) return e;                                                               \
  }

template <bool SAMPLE, int TM>
static hipError_t lmhead_packed_impl(int R, int V, int H, const void* Zp, const void* W,
                                     float* pval, int32_t* pidx, hipStream_t st, LaunchEvents ev,
                                     const DraftSampler& smp) {
  constexpr int lds = MfTile<TM, MF_N>::LDS;
  LH_ATTR((lmhead_mfma<SAMPLE, TM>), lds)
  const int n_mt = (R + TM - 1) / TM, n_nt = (V + MF_N - 1) / MF_N;
  const int per = xcd_per(n_mt * n_nt);
  DF_LAUNCH(ev.start, ev.stop, (lmhead_mfma<SAMPLE, TM>), 8 * per, MF_WAVES * 64, lds, st, R, V,
            H, (const f16_t*)Zp, (const f16_t*)W, pval, pidx, n_mt, per, smp);
  return hipGetLastError();
}

hipError_t launch_lmhead_packed(int R, int V, int H, const void* Zp, const void* W, float* pval,
                                int32_t* pidx, hipStream_t st, LaunchEvents ev, DraftSampler smp) {
  if (V % 16 || H % 32) return hipErrorInvalidValue;
  const bool rows128 = R <= 128;
  if (smp.inv_t != 0.f)
    return rows128 ? lmhead_packed_impl<true, 128>(R, V, H, Zp, W, pval, pidx, st, ev, smp)
                   : lmhead_packed_impl<true, 256>(R, V, H, Zp, W, pval, pidx, st, ev, smp);
  return rows128 ? lmhead_packed_impl<false, 128>(R, V, H, Zp, W, pval, pidx, st, ev, smp)
                 : lmhead_packed_impl<false, 256>(R, V, H, Zp, W, pval, pidx, st, ev, smp);
}

template <bool SAMPLE>
static hipError_t lmhead_argmax_impl(int dtype, int R, int V, int H, const void* Z, const void* W,
                                     float* pval, int32_t* pidx, float* logits, hipStream_t st,
                                     LaunchEvents ev, const DraftSampler& smp, float* pval2) {
  if (dtype == 0) {
    DF_LAUNCH(ev.start, ev.stop, lmhead_f32<SAMPLE>, (V + 255) / 256, 256, 0, st, R, V, H,
              (const float*)Z, (const float*)W, pval, pidx, pval2, logits, smp);
    return hipGetLastError();
  }
  if (!pval2 && lds_variant(R, H)) {
    if (V % 16 || H % 256) return hipErrorInvalidValue;
    const size_t lds = (size_t)H * 32;
    LH_ATTR((lmhead_lds<false, SAMPLE>), 160 * 1024)
    DF_LAUNCH(ev.start, ev.stop, (lmhead_lds<false, SAMPLE>), LH_GRID, LH_WAVES * 64, lds, st, R, V,
              H, (const f16_t*)Z, (const f16_t*)W, pval, pidx, logits, smp);
    return hipGetLastError();
  }
  if (H % LB_K || V % 16) return hipErrorInvalidValue;
  dim3 grid((R + LB_M - 1) / LB_M, (V + LB_N - 1) / LB_N);
  DF_LAUNCH(ev.start, ev.stop, lmhead_tiled<SAMPLE>, grid, 256, 0, st, R, V, H, (const f16_t*)Z,
            (const f16_t*)W, pval, pidx, pval2, logits, smp);
  return hipGetLastError();
}

hipError_t launch_lmhead_argmax(int dtype, int R, int V, int H, const void* Z, const void* W,
                                float* pval, int32_t* pidx, float* logits, hipStream_t st,
                                LaunchEvents ev, DraftSampler smp, float* pval2) {
  if (smp.inv_t != 0.f)
    return lmhead_argmax_impl<true>(dtype, R, V, H, Z, W, pval, pidx, logits, st, ev, smp, pval2);
  return lmhead_argmax_impl<false>(dtype, R, V, H, Z, W, pval, pidx, logits, st, ev, smp, pval2);
}

hipError_t launch_lmhead_group(int R, int V, int H, const void* Zp, const void* W, float* pval,
                               int32_t* pidx, hipStream_t st, LaunchEvents ev) {
  if (!lmhead_group_fits(R, H) || V % 16) return hipErrorInvalidValue;
  const size_t lds = (size_t)H * 32;
  LH_ATTR((lmhead_lds<true, false>), 160 * 1024)
  DF_LAUNCH(ev.start, ev.stop, (lmhead_lds<true, false>), LH_GRID, LH_WAVES * 64, lds, st, R, V, H,
            (const f16_t*)Zp, (const f16_t*)W, pval, pidx, (float*)nullptr, DraftSampler{});
  return hipGetLastError();
}

#undef LH_ATTR

hipError_t launch_argmax_reduce(int R, int ntiles, const float* pval, const int32_t* pidx,
                                int32_t* ids, int32_t* err, hipStream_t st, int R_in, int B,
                                const float* pval2, float* top2) {
  if (R <= 0) return hipSuccess;
  argmax_reduce_k<<<R, 256, 0, st>>>(B > 0 ? R_in : R, ntiles, pval, pidx, pval2, ids, B, top2,
                                     err);
  return hipGetLastError();
}
