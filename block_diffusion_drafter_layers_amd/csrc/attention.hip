// Non-causal block attention of the drafter.
//
// Every block row attends to all keys of its sequence: the injected context
// positions [0, len) and the block's own positions [len, len+B), with no mask
// inside the block ("DFlash原理深度剖析", §二.2).  q-head j reads kv-head j / G.
//
// MFMA path (bf16 storage type; split-K over the keys, flash-decoding style):
//   grid (split, kv-head, sequence); one wave per 16 query rows of the kv
//   group (G heads x B rows).  The K/V cache is fp16; Q (fp32) and the
//   probabilities are rounded to fp16 where they enter the matrix cores
//   (v_mfma_f32_16x16x32_f16, fp32 accumulation, fp32 softmax).
//   Per 64-key tile the K tile [64, d] and the transposed V tile [d, 64] are
//   staged in LDS.  Scores are computed transposed, S^T = K . Q^T, so each lane
//   owns one query column; the online softmax (exp2 domain, fp32) then needs
//   only two cross-lane shuffles, and the probabilities already sit in the
//   B-operand layout of O^T += V^T . P^T (the key order inside a 32-key step is
//   permuted identically on both operands).  Partial (o, m, l) per split are
//   merged (log-sum-exp) by a second kernel.
// fp32 path: one workgroup per (row, head), scores of a 1024-key chunk in LDS,
//   online rescaling between chunks.

#include <math.h>

#include "common.h"
#include "kernels.h"

namespace {

constexpr int AT_KT = 64;  // keys per tile

template <int D>
__global__ __launch_bounds__(512) void attn_split_mfma(DraftDims dd, const float* q,
                                                       const f16_t* kc, const f16_t* vc,
                                                       const int32_t* len, int n_split,
                                                       float* opart) {
  constexpr int KP = D + 8;       // K tile pitch (elements)
  constexpr int VP = AT_KT + 8;   // V^T tile pitch
  __shared__ __attribute__((aligned(16))) f16_t sK[AT_KT * KP];
  __shared__ __attribute__((aligned(16))) f16_t sV[D * VP];

  const int s = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nthr = blockDim.x;
  const int G = dd.Hq / dd.Hkv;
  const int B = dd.B;
  const int QD = dd.Hq * D;

  int nk = len[b] + B;
  if (nk > dd.max_ctx) nk = dd.max_ctx;
  int chunk = (nk + n_split - 1) / n_split;
  chunk = (chunk + AT_KT - 1) / AT_KT * AT_KT;
  const int k_lo = s * chunk;
  const int k_hi = min(nk, k_lo + chunk);

  // query handled by this lane (column of S^T): group row qr = 16*wave + lane%16
  const int qr = wave * 16 + (lane & 15);
  const bool qok = qr < G * B;
  const int hq = kvh * G + (qok ? qr / B : 0);
  const int rr = qok ? qr % B : 0;
  const long long qrow = (long long)b * B + rr;

  f16x8 qf[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    f16x8 h = {};
    if (qok) {
      const float* qp = q + qrow * QD + hq * D + c * 32 + (lane >> 4) * 8;
      h = cvt8(*(const floatx4*)qp, *(const floatx4*)(qp + 4));
    }
    qf[c] = h;
  }

  const float sl2 = 1.4426950408889634f / sqrtf((float)D);  // log2(e) / sqrt(d)
  float m_run = -INFINITY, l_run = 0.f;
  floatx4 oacc[D / 16];
#pragma unroll
  for (int e = 0; e < D / 16; ++e) oacc[e] = floatx4{0.f, 0.f, 0.f, 0.f};

  const f16_t* kbase = kc + ((long long)b * dd.Hkv + kvh) * dd.max_ctx * D;
  const f16_t* vbase = vc + ((long long)b * dd.Hkv + kvh) * D * (long long)dd.max_ctx;

  for (int t0 = k_lo; t0 < k_hi; t0 += AT_KT) {
    const int valid = min(AT_KT, k_hi - t0);
    // stage the K tile (rows t0..t0+63, contiguous in the cache) and the V^T tile
    // (D rows of 64 positions, positions past the end zeroed).  Both tiles have
    // NP pieces of 8 values; each thread loads up to 4 pieces of each before
    // storing, so the tile costs one memory latency.  Rows past `valid` stay
    // inside the cache (t0 is a multiple of 64 below max_ctx); their scores are
    // masked below.
    constexpr int NP = AT_KT * D / 8;
    for (int p0 = tid; p0 < NP; p0 += 4 * nthr) {
      u32x4 kv4[4], vv4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int p = min(p0 + j * nthr, NP - 1);
        kv4[j] = *(const u32x4*)(kbase + (long long)(t0 + p / (D / 8)) * D + (p % (D / 8)) * 8);
        vv4[j] = *(const u32x4*)(vbase + (long long)(p / (AT_KT / 8)) * dd.max_ctx + t0 +
                                 (p % (AT_KT / 8)) * 8);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int p = p0 + j * nthr;
        if (p < NP) {
          *(u32x4*)&sK[(p / (D / 8)) * KP + (p % (D / 8)) * 8] = kv4[j];
          const int vrow = p / (AT_KT / 8), vcol = (p % (AT_KT / 8)) * 8;
          u32x4 v = vv4[j];
          if (vcol + 8 > valid) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t keep = (vcol + 2 * e < valid ? 0xFFFFu : 0u) |
                                    (vcol + 2 * e + 1 < valid ? 0xFFFF0000u : 0u);
              v[e] &= keep;
            }
          }
          *(u32x4*)&sV[vrow * VP + vcol] = v;
        }
      }
    }
    __syncthreads();

    // S^T tile: 4 sub-tiles of 16 keys x 16 queries
    floatx4 sacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      sacc[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        const f16x8 kf = *(const f16x8*)&sK[(kt * 16 + (lane & 15)) * KP + c * 32 + (lane >> 4) * 8];
        sacc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[c], sacc[kt], 0, 0, 0);
      }
    }
    // scale, mask, tile max per query column
    float tmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kt * 16 + (lane >> 4) * 4 + i;
        float v = sacc[kt][i] * sl2;
        if (key >= valid) v = -INFINITY;
        sacc[kt][i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
    float pv[2][8];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2f(sacc[kt][i] - m_new);
        psum += p;
        pv[kt >> 1][(kt & 1) * 4 + i] = p;
      }
    const f16x8 pf[2] = {cvt8(pv[0]), cvt8(pv[1])};
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int e = 0; e < D / 16; ++e) oacc[e] *= alpha;
    // O^T += V^T . P^T ; slot j of lane group g <-> key 32h + 4g + j (j < 4), 32h + 16 + 4g + j-4
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int e = 0; e < D / 16; ++e) {
        const int off = (e * 16 + (lane & 15)) * VP + h * 32 + (lane >> 4) * 4;
        const u32x2 lo = *(const u32x2*)&sV[off], hi = *(const u32x2*)&sV[off + 16];
        const u32x4 v4 = {lo[0], lo[1], hi[0], hi[1]};
        oacc[e] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, v4), pf[h], oacc[e], 0,
                                                         0, 0);
      }
    }
    __syncthreads();
  }

  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  constexpr int SP = D + 32;  // partial slot pitch: o[D], m, l, padding
  if (qok) {
    const long long slot = ((qrow * dd.Hq + hq) * n_split + s);
    float* op = opart + slot * SP;
#pragma unroll
    for (int e = 0; e < D / 16; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i) op[e * 16 + (lane >> 4) * 4 + i] = oacc[e][i];
    if ((lane >> 4) == 0) {
      op[D] = m_run;
      op[D + 1] = l_run;
    }
  }
}

// log-sum-exp merge of the splits: one workgroup per (row, q-head), one thread per dim
template <int D>
__global__ __launch_bounds__(D) void attn_merge(DraftDims dd, int n_split, const float* opart,
                                                 float* o) {
  constexpr int SP = D + 32;
  __shared__ float sw[64];
  __shared__ float sinv;
  const int qrow = blockIdx.x, hq = blockIdx.y, e = threadIdx.x;
  const float* op = opart + ((long long)qrow * dd.Hq + hq) * n_split * SP;
  if (threadIdx.x < 64) {
    const int s = threadIdx.x;
    const float mm = s < n_split ? op[s * SP + D] : -INFINITY;
    const float ll = s < n_split ? op[s * SP + D + 1] : 0.f;
    const float mv = ll > 0.f ? mm : -INFINITY;
    const float mx = warp_max(mv);
    const float w = ll > 0.f ? exp2f(mv - mx) : 0.f;
    sw[s] = w;
    const float L = warp_sum(w * ll);
    if (s == 0) sinv = 1.f / L;
  }
  __syncthreads();
  float acc = 0.f;
  for (int s0 = 0; s0 < n_split; s0 += 8) {  // loads issued 8 at a time, summed in order
    float t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] = op[min(s0 + j, n_split - 1) * SP + e];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + j < n_split) acc += sw[s0 + j] * t[j];
  }
  o[(long long)qrow * dd.Hq * D + hq * D + e] = acc * sinv;
}

// ---- fp32 -----------------------------------------------------------------------------
constexpr int AF_CH = 1024;

__global__ __launch_bounds__(128) void attn_f32(DraftDims dd, const float* q, const float* kc,
                                                const float* vc, const int32_t* len, float* o) {
  __shared__ float sq[128];
  __shared__ float sc[AF_CH];
  __shared__ float red[16];
  const int r = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int D = dd.d, G = dd.Hq / dd.Hkv, kvh = hq / G;
  const long long qrow = (long long)b * dd.B + r;
  int nk = len[b] + dd.B;
  if (nk > dd.max_ctx) nk = dd.max_ctx;
  if (tid < D) sq[tid] = q[qrow * dd.Hq * D + hq * D + tid];
  __syncthreads();
  const float* kb = kc + ((long long)b * dd.Hkv + kvh) * dd.max_ctx * D;
  const float* vb = vc + ((long long)b * dd.Hkv + kvh) * D * (long long)dd.max_ctx;
  const float scale = 1.f / sqrtf((float)D);
  float m_run = -INFINITY, l_run = 0.f, acc = 0.f;
  for (int c0 = 0; c0 < nk; c0 += AF_CH) {
    const int n = min(AF_CH, nk - c0);
    float lmax = -INFINITY;
    for (int p = tid; p < n; p += blockDim.x) {
      const float* kr = kb + (long long)(c0 + p) * D;
      float s = 0.f;
      for (int e = 0; e < D; ++e) s = fmaf(sq[e], kr[e], s);
      s *= scale;
      sc[p] = s;
      lmax = fmaxf(lmax, s);
    }
    // block max (reuse red: negate to use block_sum-like pattern manually)
    lmax = warp_max(lmax);
    __syncthreads();
    if ((tid & 63) == 0) red[tid >> 6] = lmax;
    __syncthreads();
    float cmax = red[0];
    for (int i = 1; i < (int)(blockDim.x >> 6); ++i) cmax = fmaxf(cmax, red[i]);
    const float m_new = fmaxf(m_run, cmax);
    const float alpha = expf(m_run - m_new);
    float psum = 0.f, pacc = 0.f;
    for (int p = 0; p < n; ++p) {
      const float w = expf(sc[p] - m_new);
      psum += w;
      if (tid < D) pacc = fmaf(w, vb[(long long)tid * dd.max_ctx + c0 + p], pacc);
    }
    l_run = l_run * alpha + psum;
    acc = acc * alpha + pacc;
    m_run = m_new;
    __syncthreads();
  }
  if (tid < D) o[qrow * dd.Hq * D + hq * D + tid] = acc / l_run;
}

}  // namespace

int attention_splits(const DraftDims& dd) {
  // enough workgroups to cover the chip, but at least 256 keys per split
  const int pairs = dd.batch * dd.Hkv;
  int by_len = (dd.max_ctx + 255) / 256;
  int want = (1024 + pairs - 1) / pairs;
  int s = want < by_len ? want : by_len;
  if (s < 1) s = 1;
  if (s > 64) s = 64;  // the merge handles up to 64 splits
  return s;
}

hipError_t launch_attention(int dtype, const DraftDims& dd, const float* q, const void* kc,
                            const void* vc, const int32_t* len, int n_split, float* opart,
                            float* o, hipStream_t st, LaunchEvents ev) {
  if (dtype == 0) {
    if (dd.d > 128) return hipErrorInvalidValue;
    dim3 grid(dd.B, dd.Hq, dd.batch);
    DF_LAUNCH(ev.start, ev.stop, attn_f32, grid, 128, 0, st, dd, q, (const float*)kc, (const float*)vc,
              len, o);
    return hipGetLastError();
  }
  const int G = dd.Hq / dd.Hkv;
  const int nw = (G * dd.B + 15) / 16;
  if (nw > 8) return hipErrorInvalidValue;
  dim3 grid(n_split, dd.Hkv, dd.batch);
  if (n_split > 64) return hipErrorInvalidValue;
  dim3 mgrid(dd.batch * dd.B, dd.Hq);
  hipEvent_t none = nullptr;
  if (dd.d == 128) {
    DF_LAUNCH(ev.start, none, attn_split_mfma<128>, grid, 64 * nw, 0, st, dd, q, (const f16_t*)kc,
              (const f16_t*)vc, len, n_split, opart);
    DF_LAUNCH(none, ev.stop, attn_merge<128>, mgrid, 128, 0, st, dd, n_split, opart, o);
  } else if (dd.d == 64) {
    DF_LAUNCH(ev.start, none, attn_split_mfma<64>, grid, 64 * nw, 0, st, dd, q, (const f16_t*)kc,
              (const f16_t*)vc, len, n_split, opart);
    DF_LAUNCH(none, ev.stop, attn_merge<64>, mgrid, 64, 0, st, dd, n_split, opart, o);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
