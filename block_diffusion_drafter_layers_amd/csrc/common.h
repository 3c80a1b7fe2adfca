// Shared device helpers for the gfx950 kernels of the DFlash draft step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // bf16 kept as raw bits in memory
typedef uint16_t f16_t;   // fp16 kept as raw bits in memory

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define DF_WAVE 64

// Matrix-core operands are fp16 with fp32 accumulation.  bf16 weights are
// converted once, when packed (exact for |w| >= 2^-14; smaller values keep an
// absolute error below 2^-25).  fp32 activations are rounded to fp16 (nearest
// even) where they enter a matrix core: a relative error of 2^-11, eight times
// finer than bf16.  Values must stay within fp16 range (|x| < 65504).

__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
__device__ __forceinline__ float h2f(f16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ __forceinline__ f16_t f2h(float f) { return __builtin_bit_cast(f16_t, (_Float16)f); }

// float -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

// 8 fp32 values -> one fp16 MFMA fragment (round to nearest even)
__device__ __forceinline__ f16x8 cvt8(const floatx4 a, const floatx4 b) {
  f16x8 h;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h[j] = (_Float16)a[j];
    h[4 + j] = (_Float16)b[j];
  }
  return h;
}
__device__ __forceinline__ f16x8 cvt8(const float* x) {
  f16x8 h;
#pragma unroll
  for (int j = 0; j < 8; ++j) h[j] = (_Float16)x[j];
  return h;
}
// 8 bf16 values (raw bits) -> fp16 fragment
__device__ __forceinline__ f16x8 bf8_to_h8(const u32x4 v) {
  f16x8 h;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h[2 * j] = (_Float16)__uint_as_float(v[j] << 16);
    h[2 * j + 1] = (_Float16)__uint_as_float(v[j] & 0xFFFF0000u);
  }
  return h;
}

// Weight-streaming inner loop shared by the skinny GEMM and the lm_head.
// Weights are fragment-packed: the lane's 16 bytes of k-step t (32 k) of its
// 16-row group sit at wp + 512 t, so each load instruction of a wave reads one
// contiguous 1 KB fragment.  The A fragment of k-step t and row tile mt sits in
// LDS at sA[(t * MT + mt) * 64 + lane].  Two register buffers of U k-steps
// alternate: the loads of one are issued before the MFMAs of the other, and
// scheduling barriers keep the compiler from merging them, so 8-16 loads of
// 16 bytes stay in flight per lane.  Weights are read once: non-temporal loads.
template <int U>
__device__ __forceinline__ void load_w(f16x8 (&buf)[U], const f16_t* wp, int t0) {
#pragma unroll
  for (int u = 0; u < U; ++u) buf[u] = __builtin_nontemporal_load((const f16x8*)(wp + (t0 + u) * 512));
}

template <int U, int MT>
__device__ __forceinline__ void mma_w(const f16x8 (&buf)[U], const f16x8* sA, int lane, int t0,
                                      floatx4 (&acc)[MT]) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int slot = ((t0 + u) * MT + mt) * 64 + lane;
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(sA[slot], buf[u], acc[mt], 0, 0, 0);
    }
  }
}

// Streams the weight fragments of n_tiles work tiles (T k-steps each, T a
// multiple of U) as one continuous sequence of U-step buffers, so that loads
// stay in flight across tile boundaries.  tile_ptr(j) is the lane's fragment
// pointer of tile j at k-step 0; every tile multiplies the same A fragments
// (LDS, k-step t at slot t); done(j, acc) consumes tile j's accumulators,
// which then restart from zero.  The caller has already loaded buffer 0 of
// tile 0 into `a`.
template <int U, int MT, typename PtrF, typename DoneF>
__device__ __forceinline__ void stream_tiles(int n_tiles, int T, PtrF tile_ptr, const f16x8* sA,
                                             int lane, f16x8 (&a)[U], DoneF done) {
  const int bpt = T / U;  // buffers per tile
  const int nb = n_tiles * bpt;
  int lt = 0, lb = 1;     // next buffer to load: tile lt, buffer lb of it
  const f16_t* lp = tile_ptr(0);
  int ct = 0, cb = 0;     // buffer to multiply next
  floatx4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
  f16x8 b[U];
  auto load_next = [&](f16x8 (&buf)[U]) {
    if (lb == bpt) {
      lb = 0;
      ++lt;
      lp = tile_ptr(lt);
    }
    load_w<U>(buf, lp, lb * U);
    ++lb;
  };
  auto multiply = [&](const f16x8 (&buf)[U]) {
    mma_w<U, MT>(buf, sA, lane, cb * U, acc);
    if (++cb == bpt) {
      done(ct, acc);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
      cb = 0;
      ++ct;
    }
  };
  for (int i = 0; i < nb; i += 2) {
    if (i + 1 < nb) load_next(b);
    __builtin_amdgcn_sched_barrier(0);
    multiply(a);
    if (i + 2 < nb) load_next(a);
    __builtin_amdgcn_sched_barrier(0);
    if (i + 1 < nb) multiply(b);
  }
}

// Workgroup barrier for software pipelines fed by direct-to-LDS loads.  Each
// wave first waits (vmcnt) for exactly the loads of the stage about to be read;
// __syncthreads() would add a workgroup-scope release, which makes the compiler
// wait for every outstanding load that writes LDS -- the prefetches of the
// following stages included -- and so drains the pipeline at every step.
// Wavefront-scope fences keep the compiler from moving LDS accesses across the
// barrier without adding any wait.  LDS reads of the previous stage are complete
// by then (their values were consumed before the barrier).
__device__ __forceinline__ void barrier_pipelined() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The same barrier after this wave's own LDS stores (ds_write) have completed
// (lgkmcnt(0); vector-memory loads in flight stay in flight).
__device__ __forceinline__ void barrier_after_lds_stores() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt = 0; vmcnt, expcnt at their maxima (no wait)
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Fragment-packed fp16 K/V cache of the bf16 storage type, per (sequence, kv head):
//   K: fragment (g, c) = keys 16g.., dims 32c.. ; lane l, slot j = K[16g + l%16][32c + 8(l/16) + j]
//      (the A operand of S^T = K . Q^T), fragments ordered g-major: a 64-key tile is
//      4 * d/32 contiguous fragments.
//   V: fragment (h, e) = keys 32h.., dims 16e.. ; lane l, slot j = V[32h + key(l/16, j)][16e + l%16]
//      with key(g, j) = 4g + j (j < 4), 16 + 4g + j - 4 (j >= 4): the A operand of
//      O^T = V^T . P^T in the key order of the probabilities' registers; h-major,
//      so a 64-key tile is 2 * d/16 contiguous fragments.
// Offsets in elements from the (sequence, kv head) base; D = head dim.
__device__ __forceinline__ long long kfrag_off(int pos, int dim, int D) {
  return ((long long)(pos >> 4) * (D >> 5) + (dim >> 5)) * 512 +
         ((pos & 15) + 16 * ((dim & 31) >> 3)) * 8 + (dim & 7);
}
__device__ __forceinline__ long long vfrag_off(int pos, int dim, int D) {
  const int r = pos & 31;
  return ((long long)(pos >> 5) * (D >> 4) + (dim >> 4)) * 512 +
         ((dim & 15) + 16 * ((r & 15) >> 2)) * 8 + (r & 3) + (r >= 16 ? 4 : 0);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct Elem<bf16_t> {  // bf16_t and f16_t are both uint16_t: bf16 here
  static __device__ __forceinline__ float load(const bf16_t* p) { return bf2f(*p); }
  static __device__ __forceinline__ void store(bf16_t* p, float v) { *p = f2bf(v); }
};
// fp16 storage (the K/V cache and the lm_head rows of the bf16 storage type)
struct H16 {
  f16_t v;
};
template <> struct Elem<H16> {
  static __device__ __forceinline__ float load(const H16* p) { return h2f(p->v); }
  static __device__ __forceinline__ void store(H16* p, float x) { p->v = f2h(x); }
};

template <typename T> __device__ __forceinline__ float ld(const T* p) { return Elem<T>::load(p); }
template <typename T> __device__ __forceinline__ void st(T* p, float v) { Elem<T>::store(p, v); }

// Whether x is stored as a finite value of storage type T: fp32 any finite x;
// fp16 |x| < 65520 (from 65520 up, round-to-nearest-even gives infinity).  NaN fails.
template <typename T> __device__ __forceinline__ bool fits(float x) {
  return fabsf(x) <= 3.402823466e38f;
}
template <> __device__ __forceinline__ bool fits<H16>(float x) { return fabsf(x) < 65520.f; }

__device__ __forceinline__ float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float warp_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Block-wide sum for blockDim.x a multiple of 64 (<= 1024); `red` holds >= 16 floats.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = warp_sum(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  const int nw = blockDim.x >> 6;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

// init + sum_{s < n} p[s * stride], added in the order s = 0, 1, ..., n-1.  The
// loads are issued 8 at a time (clamped addresses, masked adds), so the sum
// costs n/8 memory latencies instead of n.
__device__ __forceinline__ float sum_strided(const float* p, long long stride, int n,
                                             float init = 0.f) {
  float v = init;
  for (int s0 = 0; s0 < n; s0 += 8) {
    float t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] = p[(long long)min(s0 + j, n - 1) * stride];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + j < n) v += t[j];
  }
  return v;
}

// Sum of n contiguous floats by one wave: lane-strided loads, then a butterfly.
__device__ __forceinline__ float wave_sum_contig(const float* p, int n, int lane) {
  float t = 0.f;
  for (int c = lane; c < n; c += 64) t += p[c];
  return warp_sum(t);
}

__device__ __forceinline__ void set_err(int32_t* err, int bits) {
  if (err) atomicOr(err, bits);
}

// cos / sin of the RoPE angle of (position, pair i): pos * theta^(-2i/d), in fp64
__device__ __forceinline__ void rope_cs(int pos, int i, int d, float theta, float& c, float& s) {
  const double inv = exp(-(2.0 * i / d) * log((double)theta));
  double sd, cd;
  sincos((double)pos * inv, &sd, &cd);
  c = (float)cd;
  s = (float)sd;
}

// Packed row p of a fuse_inject call -> (sequence, cache position), or sequence -1
// for a row no sequence owns or one past the cache (error bit 0 set).
__device__ __forceinline__ void map_row(int p, int batch, const int32_t* row_start,
                                        const int32_t* row_count, const int32_t* len, int max_ctx,
                                        int32_t* err, int& sb, int& ps) {
  sb = -1;
  ps = 0;
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
}

// len[b] += the rows of sequence b that exist in the packed buffer (clamped to max_ctx)
__device__ __forceinline__ void len_add(int b, int total_rows, const int32_t* row_start,
                                        const int32_t* row_count, int32_t* len, int max_ctx,
                                        int32_t* err) {
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

// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy
// as 1, 2, 3", SC 2011): ten rounds of two 32x32 -> 64-bit multiplies (one
// v_mad_u64_u32 each) with the published multipliers; the key is bumped by the
// published Weyl increments between rounds.  c: the counter in, the 4-word block out.
__device__ __forceinline__ void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
  constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  constexpr uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  // kept a loop: callers unroll their own loops around it, which a ten-fold
  // larger body would stop (and their register arrays would then be indexed);
  // two rounds per pass rename the words instead of moving them
#pragma unroll 2
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)M0 * c[0], p1 = (uint64_t)M1 * c[2];
    c[0] = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
    c[1] = (uint32_t)p1;
    c[2] = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
    c[3] = (uint32_t)p0;
    k0 += W0;
    k1 += W1;
  }
}
