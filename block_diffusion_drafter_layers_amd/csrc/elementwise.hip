// Row-wise kernels around the GEMMs: block embedding, split-K reduction with
// the residual add, RMSNorm application, the Q/K/V epilogue with RoPE and the
// block's cache writes, SwiGLU, the injection epilogue, and the integer
// bookkeeping (row map, len update, acceptance + trim).
//
// Activations are fp32.  T is the storage type of the weights (gains,
// embedding); the K/V cache and the rows handed to the lm_head are fp32 for
// the fp32 storage type and fp16 (H16) for bf16.  Every kernel here is
// column-parallel (a 256-column chunk or one head per workgroup), so a batch
// of 16 rows still spreads over hundreds of workgroups.
//
// RMSNorm: x * (mean(x^2) + eps)^-1/2 * g with fp32 statistics.  The reduce
// kernel leaves per-chunk partial sums of squares; the consumer (a GEMM's A
// staging or norm_rows) finishes the row statistic.
// RoPE: rotate-half pairs (i, i + d/2), angle pos * theta^(-2i/d); the angle
// and its cosine/sine are evaluated in fp64 (positions reach 32K and more,
// where an fp32 angle would already be off by ~1e-3 rad), then rounded to fp32.

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace {

// element offset of (position, dim) inside one (sequence, kv head) slice of the
// cache: plain [pos][d] K and [d][pos] V for fp32, fragment-packed for fp16
__device__ __forceinline__ long long cache_k(int pos, int dim, int D, int max_ctx, float*) {
  (void)max_ctx;
  return (long long)pos * D + dim;
}
__device__ __forceinline__ long long cache_v(int pos, int dim, int D, int max_ctx, float*) {
  (void)D;
  return (long long)dim * max_ctx + pos;
}
__device__ __forceinline__ long long cache_k(int pos, int dim, int D, int max_ctx, H16*) {
  (void)max_ctx;
  return kfrag_off(pos, dim, D);
}
__device__ __forceinline__ long long cache_v(int pos, int dim, int D, int max_ctx, H16*) {
  (void)max_ctx;
  return vfrag_off(pos, dim, D);
}

constexpr int RB = 256;       // threads per row kernel
constexpr int CB = 128;       // threads (= columns) per row-chunk kernel

// v^2 summed over each aligned run of SS_COLS lanes (one ss chunk); the lane whose
// column is a multiple of SS_COLS writes it
__device__ __forceinline__ float chunk_ss(float v) {
  float s2 = v * v;
#pragma unroll
  for (int o = 1; o < SS_COLS; o <<= 1) s2 += __shfl_xor(s2, o, 64);
  return s2;
}


// ---- block embedding --------------------------------------------------------------
__device__ __forceinline__ void unpack_bf16x8(const uint4 u, float* v) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = __uint_as_float(w[j] << 16);
    v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ void load8(const bf16_t* p, float* v) {
  unpack_bf16x8(*(const uint4*)p, v);
}
__device__ __forceinline__ void load8(const float* p, float* v) {
  const floatx4 a = *(const floatx4*)p, c = *(const floatx4*)(p + 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[j] = a[j];
    v[4 + j] = c[j];
  }
}

// One workgroup per block row; thread t owns the 8-column runs starting at
// 8 t + 8 RB h (H % 16 == 0), so each wave's loads and stores cover contiguous
// spans and a pair of neighbouring threads holds one ss chunk.  The first d/2
// threads also write the row's RoPE table.
// ids non-null: row m takes token ids[m] (a block of given tokens) instead of
// [last_tok, mask, ...].
template <typename T>
__global__ __launch_bounds__(RB) void embed_k(DraftDims dd, const int32_t* last_tok,
                                              const T* embed, int32_t* len, int32_t* base,
                                              int32_t* err, float* X, float* ss, float* rope,
                                              const int32_t* ids) {
  const int m = blockIdx.x, tid = threadIdx.x;
  const int b = m / dd.B, r = m % dd.B;
  int id = ids ? ids[m] : (r == 0 ? last_tok[b] : dd.mask_id);
  if (id < 0 || id >= dd.V) {
    if (tid == 0) set_err(err, 2);
    id = 0;
  }
  const int L = len[b] + dd.pos_off;
  if (r == 0 && tid == 0) {
    base[b] = L;
    if (L + dd.B > dd.max_ctx) set_err(err, 1);
  }
  const T* e = embed + (long long)id * dd.H;
  float* xr = X + (long long)m * dd.H;
  for (int c0 = 0; c0 < dd.H; c0 += 8 * RB) {  // uniform trip count: the shuffle below
    const int c = c0 + 8 * tid;
    const bool act = c < dd.H;
    float v[8];
    float cs = 0.f;
    if (act) {
      load8(e + c, v);
      *(floatx4*)(xr + c) = floatx4{v[0], v[1], v[2], v[3]};
      *(floatx4*)(xr + c + 4) = floatx4{v[4], v[5], v[6], v[7]};
#pragma unroll
      for (int j = 0; j < 8; ++j) cs += v[j] * v[j];
    }
    cs += __shfl_xor(cs, 1, 64);  // SS_COLS = 16 columns: two threads
    if (act && !(tid & 1)) ss[(long long)m * ss_chunks(dd.H) + c / SS_COLS] = cs;
  }
  const int half = dd.d >> 1;
  for (int i = tid; i < half; i += RB) {
    float cs, sn;
    rope_cs(L + r, i, dd.d, dd.theta, cs, sn);
    rope[((long long)m * half + i) * 2] = cs;
    rope[((long long)m * half + i) * 2 + 1] = sn;
  }
}

// One workgroup per row of a 16-row group, for the full-K QKV GEMM: as embed_k, and
// also the GEMM's packed fp16 A rows y = fp16(x * gain * sc) with the row's own
// sc = rsqrt(mean(x^2) + eps), so that y is RMSNorm(x) * gain.  Threads t < RB own
// the 16-column chunks t, t + RB, ... (H % 16 == 0); the extra wave computes the
// row's RoPE table after the row sum, beside the writes of y.

__global__ __launch_bounds__(RB + 64) void embed_group_k(DraftDims dd, const int32_t* last_tok,
                                                         const bf16_t* embed, int32_t* len,
                                                         int32_t* base, int32_t* err, float* X,
                                                         float* ss, float* rope,
                                                         const bf16_t* gain, float* sc, f16_t* y) {
  __shared__ float red[16];
  const int m = blockIdx.x, tid = threadIdx.x;
  const int b = m / dd.B, r = m % dd.B;
  int id = r == 0 ? last_tok[b] : dd.mask_id;
  if (id < 0 || id >= dd.V) {
    if (tid == 0) set_err(err, 2);
    id = 0;
  }
  const int L = len[b];
  if (r == 0 && tid == 0) {
    base[b] = L;
    if (L + dd.B > dd.max_ctx) set_err(err, 1);
  }
  const int nch = dd.H / 16;
  const bf16_t* e = embed + (long long)id * dd.H;
  float* xr = X + (long long)m * dd.H;
  float tot = 0.f;
  for (int ch = tid; tid < RB && ch < nch; ch += RB) {
    float v[16];
    unpack_bf16x8(((const uint4*)(e + ch * 16))[0], v);
    unpack_bf16x8(((const uint4*)(e + ch * 16))[1], v + 8);
    float s2 = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) s2 += v[j] * v[j];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      ((float4*)(xr + ch * 16))[j] = make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
    ss[(long long)m * nch + ch] = s2;
    tot += s2;
  }
  const float rs = rsqrtf(block_sum(tot, red) / dd.H + dd.eps);
  if (tid < RB) {
    for (int ch = tid; ch < nch; ch += RB) {
      float v[16], g[16];
      unpack_bf16x8(((const uint4*)(e + ch * 16))[0], v);
      unpack_bf16x8(((const uint4*)(e + ch * 16))[1], v + 8);
      unpack_bf16x8(((const uint4*)(gain + ch * 16))[0], g);
      unpack_bf16x8(((const uint4*)(gain + ch * 16))[1], g + 8);
#pragma unroll
      for (int h = 0; h < 2; ++h) {  // 8 consecutive k: one 16-byte run of the packed row
        const int k = ch * 16 + 8 * h;
        f16x8 o;
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = (_Float16)(v[8 * h + j] * g[8 * h + j] * rs);
        *(f16x8*)(y + (((k >> 5) * 64) + m + 16 * ((k & 31) >> 3)) * 8) = o;
      }
    }
  } else {
    const int half = dd.d >> 1;
    for (int i = tid - RB; i < half; i += 64) {
      float cs, sn;
      rope_cs(L + r, i, dd.d, dd.theta, cs, sn);
      rope[((long long)m * half + i) * 2] = cs;
      rope[((long long)m * half + i) * 2 + 1] = sn;
    }
  }
  if (tid == 0) sc[m] = rs;
}

// ---- out (+)= sum_s P[s]; ss partials ----------------------------------------------
__global__ __launch_bounds__(CB) void reduce_rows_k(int M, int N, const float* P, int S,
                                                   float* out, int accumulate, float* ss,
                                                   RowMap rm) {
  const int c = blockIdx.x, m = blockIdx.y;
  if (rm.seq && c == 0 && threadIdx.x == 0) {  // fuse_inject's row map for this row
    int sb, ps;
    map_row(rm.row0 + m, rm.batch, rm.row_start, rm.row_count, rm.len, rm.max_ctx, rm.err, sb, ps);
    rm.seq[m] = sb;
    rm.pos[m] = ps;
  }
  const int col = c * CB + threadIdx.x;
  float v = 0.f;
  if (col < N) {
    const long long i = (long long)m * N + col;
    v = sum_strided(P + i, (long long)M * N, S, accumulate ? out[i] : 0.f);
    out[i] = v;
  }
  const float s2 = chunk_ss(v);
  if (ss && col < N && col % SS_COLS == 0) ss[(long long)m * ss_chunks(N) + col / SS_COLS] = s2;
}

// ---- row-complete reduce for the batched path ---------------------------------------------
// One workgroup per row; thread t owns the 8-column runs starting at 8 t + 8 T h
// (T threads), so each wave's loads cover whole contiguous spans.  out[m] (+)=
// sum_s P[s][m] in split order, its ss partials, and -- when apack is given --
// the row RMS-normalised with `gain` as fp16 in the packed A layout of the next
// GEMM (K = N; one 16-byte store per run), so that GEMM needs no packing pass.
constexpr int RP_MAX_RUNS = 3;  // runs per thread: N <= 8 * RP_MAX_RUNS * blockDim
template <int RP_RUNS>
__global__ void reduce_pack_k(int M, int N, const float* P, int S, float* out, int accumulate,
                              float* ss, const bf16_t* gain, float eps, f16_t* apack, RowMap rm) {
  __shared__ float red[16];
  const int m = blockIdx.x, T = blockDim.x;
  if (rm.seq && threadIdx.x == 0) {  // fuse_inject's row map for this row
    int sb, ps;
    map_row(rm.row0 + m, rm.batch, rm.row_start, rm.row_count, rm.len, rm.max_ctx, rm.err, sb, ps);
    rm.seq[m] = sb;
    rm.pos[m] = ps;
  }
  const long long rowb = (long long)m * N;
  const long long MN = (long long)M * N;
  float s2 = 0.f;
  // every run's split loads are issued before any store (a store to out between them
  // would hold the next run's loads back: out and P may alias as far as the compiler
  // knows), RP_SG splits of every run at a time, added in split order
  constexpr int RP_SG = RP_RUNS == 3 ? 2 : 4;  // within the registers of a 1024-thread block
  floatx4 a[RP_RUNS], b[RP_RUNS];
#pragma unroll
  for (int h = 0; h < RP_RUNS; ++h) {
    const int c = 8 * threadIdx.x + 8 * T * h;
    const long long i = rowb + (c < N ? c : 0);
    a[h] = b[h] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (c < N && accumulate) {
      a[h] = *(const floatx4*)(out + i);
      b[h] = *(const floatx4*)(out + i + 4);
    }
  }
  for (int s0 = 0; s0 < S; s0 += RP_SG) {
    floatx4 ta[RP_RUNS][RP_SG], tb[RP_RUNS][RP_SG];
#pragma unroll
    for (int h = 0; h < RP_RUNS; ++h) {
      const int c = 8 * threadIdx.x + 8 * T * h;
      const long long i = rowb + (c < N ? c : 0);
#pragma unroll
      for (int j = 0; j < RP_SG; ++j) {
        const long long sj = (long long)min(s0 + j, S - 1) * MN + i;
        if (c < N) {
          ta[h][j] = *(const floatx4*)(P + sj);
          tb[h][j] = *(const floatx4*)(P + sj + 4);
        } else {
          ta[h][j] = tb[h][j] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
#pragma unroll
    for (int h = 0; h < RP_RUNS; ++h)
#pragma unroll
      for (int j = 0; j < RP_SG; ++j)
        if (s0 + j < S) {
          a[h] += ta[h][j];
          b[h] += tb[h][j];
        }
  }
#pragma unroll
  for (int h = 0; h < RP_RUNS; ++h) {
    const int c = 8 * threadIdx.x + 8 * T * h;
    const bool act = c < N;
    const long long i = rowb + (act ? c : 0);
    if (!act) a[h] = b[h] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (act) {
      *(floatx4*)(out + i) = a[h];
      *(floatx4*)(out + i + 4) = b[h];
    }
    // ss partial of each SS_COLS-column chunk: SS_COLS / 8 consecutive threads
    float cs = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) cs += a[h][r] * a[h][r] + b[h][r] * b[h][r];
    s2 += cs;
#pragma unroll
    for (int o = 1; o < SS_COLS / 8; o <<= 1) cs += __shfl_xor(cs, o, 64);
    if (act && (threadIdx.x & (SS_COLS / 8 - 1)) == 0)
      ss[(long long)m * (N / SS_COLS) + c / SS_COLS] = cs;
  }
  if (!apack) return;
  const float tot = block_sum(s2, red);
  const float rs = rsqrtf(tot / N + eps);
  const int KT = N / 32;
#pragma unroll
  for (int h = 0; h < RP_RUNS; ++h) {
    const int k = 8 * threadIdx.x + 8 * T * h;
    if (k >= N) break;
    const u32x4 gw = *(const u32x4*)(gain + k);
    const float v[8] = {a[h][0], a[h][1], a[h][2], a[h][3], b[h][0], b[h][1], b[h][2], b[h][3]};
    f16x8 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o[2 * j] = (_Float16)(v[2 * j] * rs * __uint_as_float(gw[j] << 16));
      o[2 * j + 1] = (_Float16)(v[2 * j + 1] * rs * __uint_as_float(gw[j] & 0xFFFF0000u));
    }
    *(f16x8*)(apack + (((long long)(m >> 4) * KT + (k >> 5)) * 64 + (m & 15) + 16 * ((k & 31) >> 3)) * 8) = o;
  }
}

// ---- y = RMSNorm(src) * g ------------------------------------------------------------
template <typename T, typename ZT>
__global__ __launch_bounds__(CB) void norm_rows_k(int N, const float* src, const float* ss,
                                                  int nc, const T* gain, float eps, ZT* z,
                                                  int compact_B, float* dbg) {
  const int c = blockIdx.x, m = blockIdx.y;
  const float t = wave_sum_contig(ss + (long long)m * nc, nc, threadIdx.x & 63);
  const float rs = rsqrtf(t / N + eps);
  const int col = c * CB + threadIdx.x;
  if (col >= N) return;
  const float v = src[(long long)m * N + col] * rs * ld(gain + col);
  if (dbg) dbg[(long long)m * N + col] = v;
  if (z) {
    if (compact_B > 0) {
      const int b = m / compact_B, r = m % compact_B;
      if (r > 0) st(z + ((long long)b * (compact_B - 1) + r - 1) * N + col, v);
    } else {
      st(z + (long long)m * N + col, v);
    }
  }
}

// ---- final-norm rows for the batched lm_head, packed ------------------------------------------
// output row mo < Mz is block row 1 + mo % (B-1) of sequence mo / (B-1); element
// (mo, col) goes to fragment (mo / 16, col / 32), lane mo % 16 + 16 (col % 32 / 8), slot col % 8
__global__ __launch_bounds__(CB) void norm_pack_k(int N, const float* src, const float* ss, int nc,
                                                  const bf16_t* gain, float eps, int B, int Mz,
                                                  f16_t* zp) {
  const int c = blockIdx.x, mo = blockIdx.y;
  const int col = c * CB + threadIdx.x;
  float v = 0.f;
  float rs = 0.f;
  int m = 0;
  if (mo < Mz) {
    m = (mo / (B - 1)) * B + 1 + mo % (B - 1);
    const float t = wave_sum_contig(ss + (long long)m * nc, nc, threadIdx.x & 63);
    rs = rsqrtf(t / N + eps);
  }
  if (col >= N) return;
  if (mo < Mz) v = src[(long long)m * N + col] * rs * bf2f(gain[col]);
  const int KT = N / 32, k = col & 31;
  const int l = (mo & 15) + 16 * (k >> 3);
  zp[(((long long)(mo >> 4) * KT + (col >> 5)) * 64 + l) * 8 + (k & 7)] = f2h(v);
}

// ---- Q/K/V epilogue of the block: one head per workgroup ------------------------------------
template <class C>
__global__ __launch_bounds__(256) void qkv_post_k(DraftDims dd, const float* P, int S,
                                                  const int32_t* len, const float* rope, float* q,
                                                  C* kc, C* vc) {
  // one thread per four consecutive dims: a RoPE item is dims i0..i0+3 and their
  // partners i0+d/2.. of one q or k head; a V item is dims e0..e0+3 of one v head
  const int m = blockIdx.x;
  const int b = m / dd.B, r = m % dd.B;
  const int pos = len[b] + dd.pos_off + r;
  const int d = dd.d, half = d >> 1;
  const int QD = dd.Hq * d, KVD = dd.Hkv * d, N = QD + 2 * KVD;
  const int M = dd.batch * dd.B;
  const float* Pm = P + (long long)m * N;
  const long long sstride = (long long)M * N;
  // the S split partials of four columns, summed in split order
  auto sum4 = [&](int col) {
    if (S == 1) return *(const floatx4*)(Pm + col);  // an unsplit GEMM's sums as they are
    floatx4 v = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < S; s0 += 4) {
      floatx4 t[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) t[j] = *(const floatx4*)(Pm + col + (long long)min(s0 + j, S - 1) * sstride);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (s0 + j < S) v += t[j];
    }
    return v;
  };
  const bool wr = pos < dd.max_ctx;
  const int n_rope = (dd.Hq + dd.Hkv) * (half / 4);
  const int t = blockIdx.y * blockDim.x + threadIdx.x;
  if (t < n_rope) {
    const int hh = t / (half / 4), i0 = (t % (half / 4)) * 4;
    const int base = hh < dd.Hq ? hh * d : QD + (hh - dd.Hq) * d;
    const floatx4 x1 = sum4(base + i0), x2 = sum4(base + half + i0);
    const float* rp = rope + ((long long)m * half + i0) * 2;  // (cos, sin) of dims i0..i0+3
    const floatx4 c01 = *(const floatx4*)rp, c23 = *(const floatx4*)(rp + 4);
    const float cs[4] = {c01[0], c01[2], c23[0], c23[2]}, sn[4] = {c01[1], c01[3], c23[1], c23[3]};
    floatx4 y1, y2;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      y1[j] = x1[j] * cs[j] - x2[j] * sn[j];
      y2[j] = x2[j] * cs[j] + x1[j] * sn[j];
    }
    if (hh < dd.Hq) {
      float* qo = q + (long long)m * QD + hh * d;
      *(floatx4*)(qo + i0) = y1;
      *(floatx4*)(qo + half + i0) = y2;
    } else if (wr) {
      C* kb = kc + ((long long)b * dd.Hkv + (hh - dd.Hq)) * dd.max_ctx * d;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        st(kb + cache_k(pos, i0 + j, d, dd.max_ctx, (C*)nullptr), y1[j]);
        st(kb + cache_k(pos, half + i0 + j, d, dd.max_ctx, (C*)nullptr), y2[j]);
      }
    }
  } else if (t < n_rope + dd.Hkv * (d / 4) && wr) {
    const int u = t - n_rope;
    const int kh = u / (d / 4), e0 = (u % (d / 4)) * 4;
    const floatx4 v = sum4(QD + KVD + kh * d + e0);
    C* vb = vc + ((long long)b * dd.Hkv + kh) * dd.max_ctx * d;
#pragma unroll
    for (int j = 0; j < 4; ++j) st(vb + cache_v(pos, e0 + j, d, dd.max_ctx, (C*)nullptr), v[j]);
  }
}

// ---- SwiGLU: out = silu(gate) * up; gate/up are column halves of P -------------------
// One thread per eight consecutive columns i0..i0+7 of a row: the gate and up split
// partials summed in split order with float4 loads, silu(gate) * up, stored as eight
// fp32 values or as one 16-byte fp16 fragment slot of the packed A rows.
__global__ void swiglu_k(int M, int I, const float* P, int S, float* out, f16_t* pout) {
  const long long total = (long long)M * (I / 8);
  const long long N = 2LL * I, MN = (long long)M * N;
  for (long long idx = blockIdx.x * (long long)blockDim.x + threadIdx.x; idx < total;
       idx += (long long)gridDim.x * blockDim.x) {
    const long long m = idx / (I / 8);
    const int i0 = (int)(idx % (I / 8)) * 8;
    const float* pm = P + m * N + i0;
    floatx4 g0 = *(const floatx4*)pm, g1 = *(const floatx4*)(pm + 4);
    floatx4 u0 = *(const floatx4*)(pm + I), u1 = *(const floatx4*)(pm + I + 4);
    for (int sp = 1; sp < S; ++sp) {
      const float* ps = pm + sp * MN;
      g0 += *(const floatx4*)ps;
      g1 += *(const floatx4*)(ps + 4);
      u0 += *(const floatx4*)(ps + I);
      u1 += *(const floatx4*)(ps + I + 4);
    }
    float v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = g0[j] / (1.f + __expf(-g0[j])) * u0[j];
      v[4 + j] = g1[j] / (1.f + __expf(-g1[j])) * u1[j];
    }
    if (pout) {  // fragment (m / 16, i0 / 32), lane m % 16 + 16 ((i0 % 32) / 8), slots 0..7
      *(f16x8*)(pout + (((m >> 4) * (I / 32) + (i0 >> 5)) * 64 + (m & 15) + 16 * ((i0 & 31) >> 3)) * 8) =
          cvt8(v);
    } else {
      *(floatx4*)(out + m * I + i0) = floatx4{v[0], v[1], v[2], v[3]};
      *(floatx4*)(out + m * I + i0 + 4) = floatx4{v[4], v[5], v[6], v[7]};
    }
  }
}

// ---- fuse_inject bookkeeping --------------------------------------------------------------
__global__ void len_update_k(int batch, int total_rows, const int32_t* row_start,
                             const int32_t* row_count, int32_t* len, int max_ctx, int32_t* err) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < batch) len_add(b, total_rows, row_start, row_count, len, max_ctx, err);
}

// injection epilogue: grid (row, layer, item chunk); one K rotation pair or one
// V element per thread
// LenUpdate (nullable): the last pass of a call also advances len (no kernel of the
// call reads len after the row map).

template <typename C>
__global__ __launch_bounds__(RB) void inject_post_k(int rows, int n_layers, int Hkv, int d,
                                                    int max_ctx, float theta, const float* P,
                                                    int S, const int32_t* seq,
                                                    const int32_t* pos, LayerPtrs cp,
                                                    LenUpdate lu) {
  if (lu.len && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
    for (int b = threadIdx.x; b < lu.batch; b += RB)
      len_add(b, lu.total_rows, lu.row_start, lu.row_count, lu.len, lu.max_ctx, lu.err);
  const int m = blockIdx.x, l = blockIdx.y;
  const int b = seq[m];
  if (b < 0) return;
  const int ps = pos[m];
  // one thread per four consecutive dims: a K item is dims i0..i0+3 and their
  // partners i0+d/2.. of one kv head, a V item dims e0..e0+3
  const int half = d >> 1, KVD = Hkv * d, N = n_layers * 2 * KVD;
  const int kitems = Hkv * half / 4;
  const int p = blockIdx.z * RB + threadIdx.x;
  if (p >= kitems + KVD / 4) return;
  const float* Pm = P + (long long)m * N + l * 2 * KVD;
  const long long sstride = (long long)rows * N;
  // the S split partials of four columns, summed in split order
  auto sum4 = [&](int col) {
    if (S == 1) return *(const floatx4*)(Pm + col);  // an unsplit GEMM's sums as they are
    floatx4 v = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < S; s0 += 4) {
      floatx4 t[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) t[j] = *(const floatx4*)(Pm + col + (long long)min(s0 + j, S - 1) * sstride);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (s0 + j < S) v += t[j];
    }
    return v;
  };
  bool ok = true;  // every value written is finite in the cache's type
  if (p < kitems) {
    const int kh = p / (half / 4), i0 = (p % (half / 4)) * 4;
    const floatx4 x1 = sum4(kh * d + i0), x2 = sum4(kh * d + i0 + half);
    C* kb = (C*)cp.k[l] + ((long long)b * Hkv + kh) * max_ctx * d;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float cs, sn;
      rope_cs(ps, i0 + j, d, theta, cs, sn);
      const float k1 = x1[j] * cs - x2[j] * sn, k2 = x2[j] * cs + x1[j] * sn;
      ok = ok && fits<C>(k1) && fits<C>(k2);
      st(kb + cache_k(ps, i0 + j, d, max_ctx, (C*)nullptr), k1);
      st(kb + cache_k(ps, i0 + j + half, d, max_ctx, (C*)nullptr), k2);
    }
  } else {
    const int vq = (p - kitems) * 4;
    const int kh = vq / d, e0 = vq % d;
    const floatx4 v = sum4(KVD + vq);
    C* vb = (C*)cp.v[l] + ((long long)b * Hkv + kh) * max_ctx * d;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ok = ok && fits<C>(v[j]);
      st(vb + cache_v(ps, e0 + j, d, max_ctx, (C*)nullptr), v[j]);
    }
  }
  if (!ok) set_err(lu.err, 8);
}


// Injection epilogue of the fp16 cache: one workgroup per (16 consecutive rows, layer,
// pair of kv heads).  The rotation frequencies are computed once per workgroup and the
// rows' (cos, sin) once per row and pair (fp64 angles, as rope_cs), in LDS, shared by
// both heads.  K: a thread takes 8 consecutive dims of one row and head and their
// partners d/2 further, so it writes two whole 16-byte slots of the packed cache (a slot
// holds 8 dims of one key).  V: a V slot holds one dim of 8 keys (keys 4g.. and
// 16 + 4g.. of a 32-key block), so the rows' values are staged in LDS as fp16 and
// written as 8-byte runs of 4 aligned consecutive positions of one sequence, single
// values where such a run is not whole inside the workgroup's rows.
constexpr int IP_ROWS = 16;
constexpr int IP_HPW = 2;      // kv heads per workgroup
constexpr int IP_MAXD = 128;   // head dims the staging covers
// Up to this many rows the per-row kernel above runs instead: it has more workgroups
// for the few rows of a round's re-injection (a batch-1 round of 16 rows measured
// 0.7227 ms with it, 0.7263 with this one; 512 rows at batch 32 alike either way); the
// bulk prefill of 8 x 32K rows spends 4.7 ms here against 14.3 ms in the per-row kernel.
constexpr int IP_SMALL_ROWS = 512;
__global__ __launch_bounds__(RB) void inject_post16_k(int rows, int n_layers, int Hkv, int d,
                                                      int max_ctx, float theta, const float* P,
                                                      int S, const int32_t* seq,
                                                      const int32_t* pos, LayerPtrs cp,
                                                      LenUpdate lu) {
  __shared__ double rinv[IP_MAXD / 2];
  __shared__ float2 rcs[IP_ROWS][IP_MAXD / 2];   // (cos, sin) per row and rotation pair
  __shared__ f16_t vst[IP_ROWS][IP_HPW * IP_MAXD];  // the V rows of the two heads, fp16
  __shared__ int rseq[IP_ROWS], rpos[IP_ROWS], rkind[IP_ROWS];
  if (lu.len && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
    for (int b = threadIdx.x; b < lu.batch; b += RB)
      len_add(b, lu.total_rows, lu.row_start, lu.row_count, lu.len, lu.max_ctx, lu.err);
  const int m0 = blockIdx.x * IP_ROWS, l = blockIdx.y, h0 = blockIdx.z * IP_HPW, tid = threadIdx.x;
  const int half = d >> 1, KVD = Hkv * d, N = n_layers * 2 * KVD;
  const int nh = min(IP_HPW, Hkv - h0);
  const long long sstride = (long long)rows * N;
  // rows: sequence and position (sequence -1: no sequence, past the cache or the rows)
  if (tid < IP_ROWS) {
    const int m = m0 + tid;
    int b = -1, ps = 0;
    if (m < rows) {
      b = seq[m];
      ps = pos[m];
      if (ps >= max_ctx) b = -1;
    }
    rseq[tid] = b;
    rpos[tid] = ps;
  }
  if (tid < half) rinv[tid] = exp(-(2.0 * tid / d) * log((double)theta));
  __syncthreads();
  // V write kind of each row: 0 none, 1 leads a whole run of 4 (positions p..p+3,
  // p % 4 == 0, one sequence, all inside these rows), 2 inside such a run, 3 single
  if (tid < IP_ROWS) {
    const int b = rseq[tid], ps = rpos[tid];
    int kind = 0;
    if (b >= 0) {
      const int lead = tid - (ps & 3);
      bool whole = lead >= 0 && lead + 3 < IP_ROWS;
      for (int j = 0; whole && j < 4; ++j)
        whole = rseq[lead + j] == b && rpos[lead + j] == ps - (ps & 3) + j;
      kind = whole ? (lead == tid ? 1 : 2) : 3;
    }
    rkind[tid] = kind;
  }
  for (int u = tid; u < IP_ROWS * half; u += RB) {
    const int i = u / half, pr = u % half;
    float c = 1.f, sn = 0.f;
    if (rseq[i] >= 0) {
      double sd, cd;
      sincos((double)rpos[i] * rinv[pr], &sd, &cd);
      c = (float)cd;
      sn = (float)sd;
    }
    rcs[i][pr] = make_float2(c, sn);
  }
  __syncthreads();
  // the S split partials of 8 consecutive columns, summed in split order
  auto sum8 = [&](const float* pm, floatx4& a, floatx4& b) {
    a = *(const floatx4*)pm;
    b = *(const floatx4*)(pm + 4);
    for (int s0 = 1; s0 < S; s0 += 4) {
      floatx4 ta[4], tb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float* q = pm + (long long)min(s0 + j, S - 1) * sstride;
        ta[j] = *(const floatx4*)q;
        tb[j] = *(const floatx4*)(q + 4);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (s0 + j < S) {
          a += ta[j];
          b += tb[j];
        }
    }
  };
  bool ok = true;  // every value written is finite in fp16
  const float* Pl = P + l * 2 * KVD;
  // K: (row, head, 8 dims of the first half) items
  const int kg = half / 8;
  for (int u = tid; u < IP_ROWS * nh * kg; u += RB) {
    const int i = u / (nh * kg), r = u % (nh * kg);
    const int b = rseq[i];
    if (b < 0) continue;
    const int kh = h0 + r / kg, i0 = (r % kg) * 8;
    const float* pm = Pl + (long long)(m0 + i) * N + kh * d + i0;
    floatx4 a1, b1, a2, b2;
    sum8(pm, a1, b1);
    sum8(pm + half, a2, b2);
    const float x1[8] = {a1[0], a1[1], a1[2], a1[3], b1[0], b1[1], b1[2], b1[3]};
    const float x2[8] = {a2[0], a2[1], a2[2], a2[3], b2[0], b2[1], b2[2], b2[3]};
    f16x8 y1, y2;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float2 t = rcs[i][i0 + j];
      const float k1 = x1[j] * t.x - x2[j] * t.y, k2 = x2[j] * t.x + x1[j] * t.y;
      ok = ok && fits<H16>(k1) && fits<H16>(k2);
      y1[j] = (_Float16)k1;
      y2[j] = (_Float16)k2;
    }
    f16_t* kb = (f16_t*)cp.k[l] + ((long long)b * Hkv + kh) * max_ctx * d;
    *(f16x8*)(kb + kfrag_off(rpos[i], i0, d)) = y1;
    *(f16x8*)(kb + kfrag_off(rpos[i], i0 + half, d)) = y2;
  }
  // V: stage the rows' values of the two heads (8 dims per item) as fp16
  const int vw = nh * d;  // staged dims per row
  for (int u = tid; u < IP_ROWS * (vw / 8); u += RB) {
    const int i = u / (vw / 8), e0 = (u % (vw / 8)) * 8;
    if (rseq[i] < 0) continue;
    floatx4 a, b;
    sum8(Pl + (long long)(m0 + i) * N + KVD + h0 * d + e0, a, b);
    f16x8 h;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ok = ok && fits<H16>(a[j]) && fits<H16>(b[j]);
      h[j] = (_Float16)a[j];
      h[4 + j] = (_Float16)b[j];
    }
    *(f16x8*)&vst[i][e0] = h;
  }
  __syncthreads();
  // V writes: (row, dim) items; a run's leader writes its 4 positions, a single row one
  for (int u = tid; u < IP_ROWS * vw; u += RB) {
    const int i = u / vw, e = u % vw;
    const int kind = rkind[i];
    if (kind == 0 || kind == 2) continue;
    const int kh = h0 + e / d, dim = e % d;
    f16_t* vb = (f16_t*)cp.v[l] + ((long long)rseq[i] * Hkv + kh) * max_ctx * d;
    const long long o = vfrag_off(rpos[i], dim, d);
    if (kind == 1) {
      const uint32_t lo = (uint32_t)vst[i][e] | ((uint32_t)vst[i + 1][e] << 16);
      const uint32_t hi = (uint32_t)vst[i + 2][e] | ((uint32_t)vst[i + 3][e] << 16);
      *(uint2*)(vb + o) = make_uint2(lo, hi);
    } else {
      vb[o] = vst[i][e];
    }
  }
  if (!ok) set_err(lu.err, 8);
}

// ---- longest matching prefix + bonus + trim: one wave per sequence ----------------------
__global__ void accept_trim_k(int batch, int B, const int32_t* drafts, const int32_t* targets,
                              int32_t* accept_len, int32_t* bonus, int32_t* len,
                              const int32_t* base, int32_t* err) {
  const int b = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (b >= batch) return;
  const bool mismatch =
      lane < B - 1 && drafts[(long long)b * (B - 1) + lane] != targets[(long long)b * B + lane];
  const unsigned long long mm = __ballot(mismatch);
  const int n = mm ? __ffsll((long long)mm) - 1 : B - 1;  // first mismatch, or all B-1 matched
  if (lane == 0) {
    accept_len[b] = n + 1;
    bonus[b] = targets[(long long)b * B + n];
    const int bs = base[b];
    if (bs < 0) {
      set_err(err, 4);
    } else {
      const int t = bs + n + 1;
      if (len[b] > t) len[b] = t;
    }
  }
}

// ---- rows of a causal pass ---------------------------------------------------------------
// The input-fusion injection feeds fused rows, not token embeddings, to the first
// layer: block row m = b B + j of pass `pos_off` takes packed fused row
// row_start[b] + pos_off + j when j + pos_off < row_count[b], else a zero row
// (padding: its outputs are never used, and its K/V land past the committed length).
// The row is the fused y RMS-normalised with the fusion gain (y_ss: y's partial
// sums of squares); also its ss partials and the RoPE table of position
// len[b] + pos_off + j.  One workgroup per block row.
template <typename T>
__global__ __launch_bounds__(RB) void gather_rows_k(DraftDims dd, const float* y, const float* y_ss,
                                                    const T* gain, const int32_t* row_start,
                                                    const int32_t* row_count, const int32_t* len,
                                                    float* X, float* ss, float* rope) {
  __shared__ float red[16];
  const int m = blockIdx.x, tid = threadIdx.x;
  const int b = m / dd.B, j = m % dd.B;
  const int nch = ss_chunks(dd.H);
  const bool real = j + dd.pos_off < row_count[b];
  const long long row = real ? (long long)row_start[b] + dd.pos_off + j : 0;
  float t = 0.f;
  if (real)
    for (int c = tid; c < nch; c += RB) t += y_ss[row * nch + c];
  const float rs = real ? rsqrtf(block_sum(t, red) / dd.H + dd.eps) : 0.f;
  float* xr = X + (long long)m * dd.H;
  for (int c0 = 0; c0 < dd.H; c0 += 8 * RB) {  // uniform trip count: the shuffle below
    const int c = c0 + 8 * tid;
    const bool act = c < dd.H;
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float cs = 0.f;
    if (act) {
      if (real) {
        float g[8];
        load8(y + row * dd.H + c, v);
        load8(gain + c, g);
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] *= rs * g[k];
      }
      *(floatx4*)(xr + c) = floatx4{v[0], v[1], v[2], v[3]};
      *(floatx4*)(xr + c + 4) = floatx4{v[4], v[5], v[6], v[7]};
#pragma unroll
      for (int k = 0; k < 8; ++k) cs += v[k] * v[k];
    }
    cs += __shfl_xor(cs, 1, 64);
    if (act && !(tid & 1)) ss[(long long)m * nch + c / SS_COLS] = cs;
  }
  const int half = dd.d >> 1;
  const int L = len[b] + dd.pos_off;
  for (int i = tid; i < half; i += RB) {
    float c, sn;
    rope_cs(L + j, i, dd.d, dd.theta, c, sn);
    rope[((long long)m * half + i) * 2] = c;
    rope[((long long)m * half + i) * 2 + 1] = sn;
  }
}

// len[b] += add, clamped to max_ctx (overflow bit)
__global__ void len_add_k(int batch, int add, int32_t* len, int max_ctx, int32_t* err) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  int nl = len[b] + add;
  if (nl > max_ctx) {
    set_err(err, 1);
    nl = max_ctx;
  }
  len[b] = nl;
}

// out[m][c] = X[m][c] in the storage type (the hidden states a pass hands out)
template <typename T>
__global__ void store_rows_k(long long n8, const float* X, T* out) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n8;
       i += (long long)gridDim.x * blockDim.x) {
    float v[8];
    load8(X + 8 * i, v);
#pragma unroll
    for (int k = 0; k < 8; ++k) st(out + 8 * i + k, v[k]);
  }
}

}  // namespace

// four-dim items of the injection epilogue: K pairs of dims (i0.., i0 + d/2..), then V
inline int n_kv_items(int Hkv, int d) { return Hkv * (d / 2) / 4 + Hkv * d / 4; }

#define DISPATCH_T(dtype, ...)                 \
  if ((dtype) == 0) {                           \
    using T = float;                            \
    __VA_ARGS__;                                \
  } else {                                      \
    using T = bf16_t;                           \
    __VA_ARGS__;                                \
  }

hipError_t launch_gather_rows(int dtype, const DraftDims& dd, const float* y, const float* y_ss,
                              const void* gain, const int32_t* row_start,
                              const int32_t* row_count, const int32_t* len, float* X, float* ss,
                              float* rope, hipStream_t st) {
  if (dd.H % 16) return hipErrorInvalidValue;
  DISPATCH_T(dtype, gather_rows_k<T><<<dd.batch * dd.B, RB, 0, st>>>(dd, y, y_ss, (const T*)gain,
                                                                      row_start, row_count, len, X,
                                                                      ss, rope));
  return hipGetLastError();
}

hipError_t launch_len_add(int batch, int add, int32_t* len, int max_ctx, int32_t* err,
                          hipStream_t st) {
  len_add_k<<<(batch + 255) / 256, 256, 0, st>>>(batch, add, len, max_ctx, err);
  return hipGetLastError();
}

hipError_t launch_store_rows(int dtype, int M, int H, const float* X, void* out, hipStream_t st) {
  if (H % 8) return hipErrorInvalidValue;
  const long long n8 = (long long)M * H / 8;
  const int blocks = (int)std::min<long long>((n8 + 255) / 256, 4096);
  DISPATCH_T(dtype, store_rows_k<T><<<blocks, 256, 0, st>>>(n8, X, (T*)out));
  return hipGetLastError();
}

hipError_t launch_embed(int dtype, const DraftDims& dd, const int32_t* last_tok, const void* embed,
                        int32_t* len, int32_t* base, int32_t* err, float* X, float* ss,
                        float* rope, hipStream_t st, const void* gain, float* sc, void* y,
                        const int32_t* ids) {
  if (y) {  // one 16-row group, bf16 storage
    const int M = dd.batch * dd.B;
    if (dtype == 0 || M > 16 || dd.H % 16 || !gain || !sc || ids || dd.pos_off) return hipErrorInvalidValue;
    embed_group_k<<<M, RB + 64, 0, st>>>(dd, last_tok, (const bf16_t*)embed, len, base, err, X, ss, rope,
                                    (const bf16_t*)gain, sc, (f16_t*)y);
    return hipGetLastError();
  }
  if (dd.H % 16) return hipErrorInvalidValue;
  DISPATCH_T(dtype, embed_k<T><<<dd.batch * dd.B, RB, 0, st>>>(dd, last_tok, (const T*)embed, len,
                                                                  base, err, X, ss, rope, ids));
  return hipGetLastError();
}

hipError_t launch_reduce_rows(int M, int N, const float* P, int S, float* out, bool accumulate,
                              float* ss, hipStream_t st, const RowMap* rm) {
  if (M == 0) return hipSuccess;
  dim3 grid((N + CB - 1) / CB, M);
  reduce_rows_k<<<grid, CB, 0, st>>>(M, N, P, S, out, accumulate ? 1 : 0, ss,
                                     rm ? *rm : RowMap{});
  return hipGetLastError();
}

hipError_t launch_reduce_pack(int M, int N, const float* P, int S, float* out, bool accumulate,
                              float* ss, const void* gain, float eps, void* apack,
                              hipStream_t st, const RowMap* rm) {
  if (M == 0) return hipSuccess;
  // ~16 columns per thread in whole waves; at most RP_MAX_RUNS runs of 8 each
  int threads = (N / 16 + 63) / 64 * 64;
  while (8 * RP_MAX_RUNS * threads < N) threads += 64;
  if (N % 256 || threads > 1024 || S < 1) return hipErrorInvalidValue;
  const int runs = (N + 8 * threads - 1) / (8 * threads);
  const RowMap map = rm ? *rm : RowMap{};
#define RP_LAUNCH(R)                                                                            \
  reduce_pack_k<R><<<M, threads, 0, st>>>(M, N, P, S, out, accumulate ? 1 : 0, ss,               \
                                          (const bf16_t*)gain, eps, (f16_t*)apack, map)
  if (runs == 1) RP_LAUNCH(1);
  else if (runs == 2) RP_LAUNCH(2);
  else RP_LAUNCH(3);
#undef RP_LAUNCH
  return hipGetLastError();
}

hipError_t launch_norm_rows(int dtype, int M, int N, const float* src, const float* ss,
                            int ss_nch, const void* gain, float eps, void* z, int compact_B,
                            float* dbg, hipStream_t st) {
  if (M == 0) return hipSuccess;
  dim3 grid((N + CB - 1) / CB, M);
  if (dtype == 0)
    norm_rows_k<float, float><<<grid, CB, 0, st>>>(N, src, ss, ss_nch, (const float*)gain, eps,
                                                   (float*)z, compact_B, dbg);
  else
    norm_rows_k<bf16_t, H16><<<grid, CB, 0, st>>>(N, src, ss, ss_nch, (const bf16_t*)gain, eps,
                                                  (H16*)z, compact_B, dbg);
  return hipGetLastError();
}

hipError_t launch_norm_pack(const DraftDims& dd, const float* src, const float* ss, int ss_nch,
                            const void* gain, int Mpad, void* zp, hipStream_t st) {
  const int Mz = dd.batch * (dd.B - 1);
  if (Mpad < Mz || Mpad % 16 || dd.H % 32) return hipErrorInvalidValue;
  dim3 grid((dd.H + CB - 1) / CB, Mpad);
  norm_pack_k<<<grid, CB, 0, st>>>(dd.H, src, ss, ss_nch, (const bf16_t*)gain, dd.eps, dd.B, Mz,
                                   (f16_t*)zp);
  return hipGetLastError();
}

hipError_t launch_qkv_post(int dtype, const DraftDims& dd, const float* P, int S,
                           const int32_t* len, const float* rope, float* q, void* kc, void* vc,
                           hipStream_t st) {
  if (dd.d % 8) return hipErrorInvalidValue;  // four-dim items of each half of a head
  const int items = (dd.Hq + dd.Hkv) * (dd.d / 8) + dd.Hkv * (dd.d / 4);
  dim3 grid(dd.batch * dd.B, (items + 255) / 256);
  if (dtype == 0)
    qkv_post_k<float><<<grid, 256, 0, st>>>(dd, P, S, len, rope, q, (float*)kc, (float*)vc);
  else
    qkv_post_k<H16><<<grid, 256, 0, st>>>(dd, P, S, len, rope, q, (H16*)kc, (H16*)vc);
  return hipGetLastError();
}

hipError_t launch_swiglu(int M, int I, const float* P, int S, float* out, hipStream_t st,
                         uint16_t* pout) {
  const long long total = (long long)M * (I / 8);
  if (I % 8 || (pout && I % 32)) return hipErrorInvalidValue;
  int blocks = (int)((total + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  swiglu_k<<<blocks, 256, 0, st>>>(M, I, P, S, out, (f16_t*)pout);
  return hipGetLastError();
}

hipError_t launch_inject_post(int dtype, int rows, int n_layers, int Hkv, int d, int max_ctx,
                              float theta, const float* P, int S, const int32_t* seq,
                              const int32_t* pos, void* const* kcs, void* const* vcs,
                              hipStream_t st, int batch, int total_rows, const int32_t* row_start,
                              const int32_t* row_count, int32_t* len, int32_t* err) {
  LenUpdate lu{batch, total_rows, max_ctx, row_start, row_count, len, err};
  if (rows == 0) return hipSuccess;
  if (n_layers > DF_MAX_LAYERS) return hipErrorInvalidValue;
  LayerPtrs cp;
  for (int l = 0; l < n_layers; ++l) {
    cp.k[l] = kcs[l];
    cp.v[l] = vcs[l];
  }
  if (d % 8) return hipErrorInvalidValue;
  const int items = n_kv_items(Hkv, d);
  dim3 grid(rows, n_layers, (items + RB - 1) / RB);
  if (dtype == 0) {
    inject_post_k<float><<<grid, RB, 0, st>>>(rows, n_layers, Hkv, d, max_ctx, theta, P, S, seq, pos,
                                              cp, lu);
  } else if (rows <= IP_SMALL_ROWS) {  // a round's re-injection: one workgroup per row and layer
    inject_post_k<H16><<<grid, RB, 0, st>>>(rows, n_layers, Hkv, d, max_ctx, theta, P, S, seq, pos,
                                            cp, lu);
  } else {
    if (d % 16 || d > IP_MAXD) return hipErrorInvalidValue;
    const dim3 g16((rows + IP_ROWS - 1) / IP_ROWS, n_layers, (Hkv + IP_HPW - 1) / IP_HPW);
    inject_post16_k<<<g16, RB, 0, st>>>(rows, n_layers, Hkv, d, max_ctx, theta, P, S, seq, pos, cp,
                                        lu);
  }
  return hipGetLastError();
}

hipError_t launch_len_update(int batch, int total_rows, const int32_t* row_start,
                             const int32_t* row_count, int32_t* len, int max_ctx, int32_t* err,
                             hipStream_t st) {
  len_update_k<<<(batch + 255) / 256, 256, 0, st>>>(batch, total_rows, row_start, row_count, len,
                                                    max_ctx, err);
  return hipGetLastError();
}

hipError_t launch_accept_trim(int batch, int B, const int32_t* drafts, const int32_t* targets,
                              int32_t* accept_len, int32_t* bonus, int32_t* len,
                              const int32_t* base, int32_t* err, hipStream_t st) {
  const int wpb = 4;
  accept_trim_k<<<(batch + wpb - 1) / wpb, 64 * wpb, 0, st>>>(batch, B, drafts, targets,
                                                              accept_len, bonus, len, base, err);
  return hipGetLastError();
}
