// Row-wise kernels around the GEMMs: block embedding, residual + RMSNorm,
// fusion RMSNorm, Q/K/V epilogue with RoPE and cache writes, SwiGLU, the
// injection epilogue, and the integer bookkeeping (row map, len update,
// acceptance + trim).
//
// RMSNorm: x * (mean(x^2) + eps)^-1/2 * g with fp32 statistics.
// RoPE: rotate-half pairs (i, i + d/2), angle pos * theta^(-2i/d); the angle
// and its cosine/sine are evaluated in fp64 (positions reach 32K and more,
// where an fp32 angle would already be off by ~1e-3 rad), then rounded to fp32.

#include "common.h"
#include "kernels.h"

namespace {

constexpr int RB = 256;  // threads per row kernel

// ---- block embedding + first RMSNorm --------------------------------------------
template <typename T>
__global__ __launch_bounds__(RB) void embed_norm_k(DraftDims dd, const int32_t* last_tok,
                                                   const T* embed, const T* gain, int32_t* len,
                                                   int32_t* base, int32_t* err, float* X, T* h) {
  __shared__ float red[16];
  const int m = blockIdx.x;
  const int b = m / dd.B, r = m % dd.B;
  int id = r == 0 ? last_tok[b] : dd.mask_id;
  if (id < 0 || id >= dd.V) {
    if (threadIdx.x == 0) set_err(err, 2);
    id = 0;
  }
  if (r == 0 && threadIdx.x == 0) {
    const int L = len[b];
    base[b] = L;
    if (L + dd.B > dd.max_ctx) set_err(err, 1);
  }
  const T* e = embed + (long long)id * dd.H;
  float* x = X + (long long)m * dd.H;
  float ss = 0.f;
  for (int i = threadIdx.x; i < dd.H; i += RB) {
    const float v = ld(e + i);
    x[i] = v;
    ss += v * v;
  }
  ss = block_sum(ss, red);
  const float rs = rsqrtf(ss / dd.H + dd.eps);
  T* o = h + (long long)m * dd.H;
  for (int i = threadIdx.x; i < dd.H; i += RB) st(o + i, x[i] * rs * ld(gain + i));
}

// ---- X += sum_s P[s]; out = RMSNorm(X) * g ------------------------------------------
template <typename T>
__global__ __launch_bounds__(RB) void residual_norm_k(int M, int H, const float* P, int S,
                                                      float* X, const T* gain, float eps,
                                                      T* out, int compact_B, float* dbg) {
  __shared__ float red[16];
  const int m = blockIdx.x;
  float* x = X + (long long)m * H;
  float ss = 0.f;
  for (int i = threadIdx.x; i < H; i += RB) {
    float v = x[i];
    for (int s = 0; s < S; ++s) v += P[((long long)s * M + m) * H + i];
    x[i] = v;
    ss += v * v;
  }
  ss = block_sum(ss, red);
  const float rs = rsqrtf(ss / H + eps);
  T* o = nullptr;
  if (compact_B > 0) {
    const int b = m / compact_B, r = m % compact_B;
    if (r > 0) o = out + ((long long)b * (compact_B - 1) + r - 1) * H;
  } else {
    o = out + (long long)m * H;
  }
  float* dg = dbg ? dbg + (long long)m * H : nullptr;
  for (int i = threadIdx.x; i < H; i += RB) {
    const float v = x[i] * rs * ld(gain + i);
    if (o) st(o + i, v);
    if (dg) dg[i] = v;
  }
}

// ---- fusion: c = RMSNorm(sum_s P[s]) * g -----------------------------------------------
template <typename T>
__global__ __launch_bounds__(RB) void fuse_norm_k(int M, int H, const float* P, int S,
                                                  const T* gain, float eps, T* out, float* dbg) {
  __shared__ float red[16];
  extern __shared__ float row[];
  const int m = blockIdx.x;
  float ss = 0.f;
  for (int i = threadIdx.x; i < H; i += RB) {
    float v = 0.f;
    for (int s = 0; s < S; ++s) v += P[((long long)s * M + m) * H + i];
    row[i] = v;
    ss += v * v;
  }
  ss = block_sum(ss, red);
  const float rs = rsqrtf(ss / H + eps);
  for (int i = threadIdx.x; i < H; i += RB) {
    const float v = row[i] * rs * ld(gain + i);
    st(out + (long long)m * H + i, v);
    if (dbg) dbg[(long long)m * H + i] = v;
  }
}

// cos/sin of pos * theta^(-2i/d), i < d/2, into LDS (fp64 evaluation).
__device__ __forceinline__ void rope_table(float* cs, float* sn, int pos, int d, float theta) {
  const int half = d >> 1;
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    const double inv = exp(-(2.0 * i / d) * log((double)theta));
    double s, c;
    sincos((double)pos * inv, &s, &c);
    cs[i] = (float)c;
    sn[i] = (float)s;
  }
}

// ---- Q/K/V epilogue of the block: RoPE on Q and K, K/V into the cache tail ------------
template <typename T>
__global__ __launch_bounds__(RB) void qkv_post_k(DraftDims dd, const float* P, int S,
                                                 const int32_t* len, T* q, T* kc, T* vc) {
  __shared__ float cs[64], sn[64];
  const int m = blockIdx.x;
  const int b = m / dd.B, r = m % dd.B;
  const int pos = len[b] + r;
  const int d = dd.d, half = d >> 1;
  const int QD = dd.Hq * d, KVD = dd.Hkv * d, N = QD + 2 * KVD;
  const int M = dd.batch * dd.B;
  rope_table(cs, sn, pos, d, dd.theta);
  __syncthreads();
  auto sumP = [&](int col) {
    float v = 0.f;
    for (int s = 0; s < S; ++s) v += P[((long long)s * M + m) * N + col];
    return v;
  };
  const bool wr = pos < dd.max_ctx;
  // rotary pairs of the Hq query heads and Hkv key heads
  const int npairs = (dd.Hq + dd.Hkv) * half;
  for (int p = threadIdx.x; p < npairs; p += RB) {
    const int hh = p / half, i = p % half;
    const int col = hh < dd.Hq ? hh * d + i : QD + (hh - dd.Hq) * d + i;
    const float x1 = sumP(col), x2 = sumP(col + half);
    const float y1 = x1 * cs[i] - x2 * sn[i];
    const float y2 = x2 * cs[i] + x1 * sn[i];
    if (hh < dd.Hq) {
      T* qo = q + (long long)m * QD + hh * d;
      st(qo + i, y1);
      st(qo + i + half, y2);
    } else if (wr) {
      const int kh = hh - dd.Hq;
      T* ko = kc + (((long long)b * dd.Hkv + kh) * dd.max_ctx + pos) * d;
      st(ko + i, y1);
      st(ko + i + half, y2);
    }
  }
  if (!wr) return;
  for (int p = threadIdx.x; p < KVD; p += RB) {
    const int kh = p / d, e = p % d;
    const float v = sumP(QD + KVD + p);
    st(vc + (((long long)b * dd.Hkv + kh) * d + e) * dd.max_ctx + pos, v);
  }
}

// ---- SwiGLU: out = silu(gate) * up; gate/up are column halves of P -------------------
template <typename T>
__global__ void swiglu_k(int M, int I, const float* P, int S, T* out) {
  const long long total = (long long)M * I;
  const long long N = 2LL * I;
  for (long long idx = blockIdx.x * (long long)blockDim.x + threadIdx.x; idx < total;
       idx += (long long)gridDim.x * blockDim.x) {
    const long long m = idx / I, i = idx % I;
    float g = 0.f, u = 0.f;
    for (int s = 0; s < S; ++s) {
      const float* ps = P + ((long long)s * M + m) * N;
      g += ps[i];
      u += ps[I + i];
    }
    st(out + idx, g / (1.f + __expf(-g)) * u);
  }
}

// ---- fuse_inject bookkeeping --------------------------------------------------------------
__global__ void rowmap_k(int total_rows, int batch, const int32_t* row_start,
                         const int32_t* row_count, const int32_t* len, int max_ctx,
                         int32_t* seq, int32_t* pos, int32_t* err) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= total_rows) return;
  int sb = -1, ps = 0;
  for (int b = 0; b < batch; ++b) {
    const int a = row_start[b], c = row_count[b];
    if (a >= 0 && c > 0 && p >= a && p < a + c) {
      sb = b;
      ps = len[b] + (p - a);
      break;
    }
  }
  if (sb >= 0 && ps >= max_ctx) {
    set_err(err, 1);
    sb = -1;
  }
  seq[p] = sb;
  pos[p] = ps;
}

template <typename T>
__global__ __launch_bounds__(RB) void inject_post_k(int rows, int n_layers, int Hkv, int d,
                                                    int max_ctx, float theta, const float* P,
                                                    int S, const int32_t* seq,
                                                    const int32_t* pos, LayerPtrs cp) {
  __shared__ float cs[64], sn[64];
  const int m = blockIdx.x;
  const int b = seq[m];
  if (b < 0) return;
  const int ps = pos[m];
  const int half = d >> 1, KVD = Hkv * d, N = n_layers * 2 * KVD;
  rope_table(cs, sn, ps, d, theta);
  __syncthreads();
  auto sumP = [&](int col) {
    float v = 0.f;
    for (int s = 0; s < S; ++s) v += P[((long long)s * rows + m) * N + col];
    return v;
  };
  const int kpairs = Hkv * half;
  for (int p = threadIdx.x; p < n_layers * (kpairs + KVD); p += RB) {
    const int l = p / (kpairs + KVD), q = p % (kpairs + KVD);
    const int cbase = l * 2 * KVD;
    if (q < kpairs) {
      const int kh = q / half, i = q % half;
      const float x1 = sumP(cbase + kh * d + i), x2 = sumP(cbase + kh * d + i + half);
      T* ko = (T*)cp.k[l] + (((long long)b * Hkv + kh) * max_ctx + ps) * d;
      st(ko + i, x1 * cs[i] - x2 * sn[i]);
      st(ko + i + half, x2 * cs[i] + x1 * sn[i]);
    } else {
      const int vq = q - kpairs;
      const int kh = vq / d, e = vq % d;
      st((T*)cp.v[l] + (((long long)b * Hkv + kh) * d + e) * max_ctx + ps, sumP(cbase + KVD + vq));
    }
  }
}

__global__ void len_update_k(int batch, int total_rows, const int32_t* row_start,
                             const int32_t* row_count, int32_t* len, int max_ctx, int32_t* err) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  // only rows that exist in the packed buffer count
  int add = row_count[b];
  const int avail = total_rows - row_start[b];
  if (add > avail) add = avail;
  if (add < 0 || row_start[b] < 0) add = 0;
  int nl = len[b] + add;
  if (nl > max_ctx) {
    set_err(err, 1);
    nl = max_ctx;
  }
  len[b] = nl;
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

}  // namespace

#define DISPATCH_T(dtype, ...)                 \
  if ((dtype) == 0) {                           \
    using T = float;                            \
    __VA_ARGS__;                                \
  } else {                                      \
    using T = bf16_t;                           \
    __VA_ARGS__;                                \
  }

hipError_t launch_embed_norm(int dtype, const DraftDims& dd, const int32_t* last_tok,
                             const void* embed, const void* gain, int32_t* len, int32_t* base,
                             int32_t* err, float* X, void* h, hipStream_t st) {
  DISPATCH_T(dtype, embed_norm_k<T><<<dd.batch * dd.B, RB, 0, st>>>(
                        dd, last_tok, (const T*)embed, (const T*)gain, len, base, err, X, (T*)h));
  return hipGetLastError();
}

hipError_t launch_residual_norm(int dtype, int M, int H, const float* P, int S, float* X,
                                const void* gain, float eps, void* out, int compact_B,
                                float* dbg, hipStream_t st) {
  DISPATCH_T(dtype, residual_norm_k<T><<<M, RB, 0, st>>>(M, H, P, S, X, (const T*)gain, eps,
                                                         (T*)out, compact_B, dbg));
  return hipGetLastError();
}

hipError_t launch_fuse_norm(int dtype, int M, int H, const float* P, int S, const void* gain,
                            float eps, void* out, float* dbg, hipStream_t st) {
  if (M == 0) return hipSuccess;
  DISPATCH_T(dtype, fuse_norm_k<T><<<M, RB, H * sizeof(float), st>>>(M, H, P, S, (const T*)gain,
                                                                     eps, (T*)out, dbg));
  return hipGetLastError();
}

hipError_t launch_qkv_post(int dtype, const DraftDims& dd, const float* P, int S,
                           const int32_t* len, void* q, void* kc, void* vc, int32_t* err,
                           hipStream_t st) {
  (void)err;
  DISPATCH_T(dtype, qkv_post_k<T><<<dd.batch * dd.B, RB, 0, st>>>(dd, P, S, len, (T*)q, (T*)kc,
                                                                  (T*)vc));
  return hipGetLastError();
}

hipError_t launch_swiglu(int dtype, int M, int I, const float* P, int S, void* out,
                         hipStream_t st) {
  const long long total = (long long)M * I;
  int blocks = (int)((total + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  DISPATCH_T(dtype, swiglu_k<T><<<blocks, 256, 0, st>>>(M, I, P, S, (T*)out));
  return hipGetLastError();
}

hipError_t launch_rowmap(int total_rows, int batch, const int32_t* row_start,
                         const int32_t* row_count, const int32_t* len, int max_ctx,
                         int32_t* seq, int32_t* pos, int32_t* err, hipStream_t st) {
  rowmap_k<<<(total_rows + 255) / 256, 256, 0, st>>>(total_rows, batch, row_start, row_count,
                                                     len, max_ctx, seq, pos, err);
  return hipGetLastError();
}

hipError_t launch_inject_post(int dtype, int rows, int n_layers, int Hkv, int d, int max_ctx,
                              float theta, const float* P, int S, const int32_t* seq,
                              const int32_t* pos, void* const* kcs, void* const* vcs,
                              hipStream_t st) {
  if (rows == 0) return hipSuccess;
  if (n_layers > DF_MAX_LAYERS) return hipErrorInvalidValue;
  LayerPtrs cp;
  for (int l = 0; l < n_layers; ++l) {
    cp.k[l] = kcs[l];
    cp.v[l] = vcs[l];
  }
  DISPATCH_T(dtype, inject_post_k<T><<<rows, RB, 0, st>>>(rows, n_layers, Hkv, d, max_ctx, theta,
                                                          P, S, seq, pos, cp));
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
