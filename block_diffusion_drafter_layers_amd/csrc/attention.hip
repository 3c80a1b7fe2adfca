// Non-causal block attention of the drafter.
//
// Every block row attends to all keys of its sequence: the injected context
// positions [0, len) and the block's own positions [len, len+B), with no mask
// inside the block ("DFlash原理深度剖析", §二.2).  q-head j reads kv-head j / G.
//
// MFMA path (bf16 storage type; split-K over the keys, flash-decoding style):
//   one wave per 16 query rows of the kv group (G heads x B rows), at least 4.
//   The K/V cache is fp16 in the fragment-packed layout (common.h): a 64-key
//   tile of K and of V is 16 contiguous 1 KB fragments each, already in MFMA
//   operand order, so the tiles stream into LDS with 16-byte direct-to-LDS
//   loads, double-buffered, and are read back conflict-free.  Q (fp32, times the
//   score scale) and the probabilities are rounded to fp16 where they enter the
//   matrix cores (v_mfma_f32_16x16x32_f16, fp32 accumulation, fp32 softmax).  Scores are
//   computed transposed, S^T = K . Q^T, so each lane owns one query column; the
//   online softmax (exp2 domain) then needs only two cross-lane shuffles, and
//   the probabilities already sit in the B-operand layout of O^T += V^T . P^T
//   (the V fragments hold the keys in the same permuted order).  Partial
//   (o, m, l) per key range are merged (log-sum-exp) by a second kernel.
//   Two ways of cutting the keys:
//   - one 16-row block (batch 1): at most 32 chunks of whole 64-key tiles per
//     sequence, their length set on the device from the sequence's length, grid
//     (kv-head, split, sequence), so the merge finds its partials without a lookup;
//   - batched steps: 512 workgroups each take an equal share of all the
//     (sequence, kv head, tile) work laid end to end, whatever the mix of
//     context lengths; the merge finds a segment's pieces in a small table.
// fp32 path: one workgroup per (row, head), scores of a 1024-key chunk in LDS,
//   online rescaling between chunks.

#include <math.h>

#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace {

constexpr int AT_CHUNK_UNIT = 64;  // split chunks are whole multiples of this many keys
constexpr int AT_MAX_SPLIT = 128;  // splits the merge handles (a multiple of the head dim)
// Fixed-chunk split: a sequence's keys are cut into at most this many chunks of whole
// 64-key tiles, the chunk length following the sequence's own length (known on the
// device only).  Measured per layer (split + merge, one 16-row block): 1024 keys, 17
// chunks of 64 15.2 us, 9 of 128 15.6, 5 of 256 18.1; 4000 keys, 63 of 64 24.7, 32 of 128
// 18.1, 16 of 256 19.2: past ~32 chunks the merge's reads and the workgroups' start-ups
// cost more than the parallelism gives.
constexpr int AT_FIXED_SPLITS = 32;
// Virtual tiles the balanced split charges for each piece a workgroup starts (the
// piece's Q, its pipeline's first tile, its partial's stores), so that workgroups
// whose share crosses segments stream fewer tiles.  Measured per layer at batch 32
// with contexts of 705..8144 keys (two passes each): 0 (tiles alone) 126.0 us, 2 123.4,
// 3 122.7, 4 122.5; at 8 x 32K 172.9 -> 171.9 with 2.
constexpr int AT_PIECE_COST = 3;
static_assert(AT_FIXED_SPLITS <= AT_MAX_SPLIT, "the merge's split capacity");
__device__ __forceinline__ int fixed_chunk(int nk, int n_split) {
  const int tiles = (nk + AT_CHUNK_UNIT - 1) / AT_CHUNK_UNIT;
  // n_split is AT_FIXED_SPLITS unless max_ctx is short: a shift instead of a division
  // on the way to the first load
  const int per = n_split == AT_FIXED_SPLITS ? (tiles + AT_FIXED_SPLITS - 1) / AT_FIXED_SPLITS
                                             : (tiles + n_split - 1) / n_split;
  return AT_CHUNK_UNIT * per;
}

typedef __attribute__((address_space(3))) void lds_void;
// cache-policy operand of a load: non-temporal (streamed once, low retention)
constexpr int AT_CPOL_NT = 2;

// wait until at most n vector-memory operations of this wave are outstanding
// (n a multiple of FPW up to 3 FPW)
template <int FPW>
__device__ __forceinline__ void vm_wait_tiles(int tiles) {
  auto w = [](auto c) {
    constexpr int N = decltype(c)::value;
    static_assert(N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  };
  if (tiles <= 0) w(std::integral_constant<int, 0>{});
  else if (tiles == 1) w(std::integral_constant<int, FPW>{});
  else if (tiles == 2) w(std::integral_constant<int, 2 * FPW>{});
  else w(std::integral_constant<int, 3 * FPW>{});
}

// 2^x for the online softmax, whose exponents are <= 0: the bare v_exp_f32 (a result
// below 2^-126 becomes 0, which no weight in (0, 1] notices); the library exp2f adds
// five instructions per call to keep subnormal results.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max over lanes l, l^16, l^32 and l^48 (the four 16-lane rows at one position): a
// row swap then a half swap (v_permlane16_swap, v_permlane32_swap), two VALU
// instructions instead of two LDS-crossbar permutes on the softmax's critical path.
// Each swap's two results pass through an empty asm statement before the max: given
// the same value in both operands, the compiler otherwise folds the max of the two
// results into the first one alone (a max over part of the column, measured).  A
// wrong max leaves the softmax exact (it cancels) until a probability exceeds the
// fp16 range of the P.V product, where it becomes inf.
__device__ __forceinline__ float swap_max(unsigned r0, unsigned r1) {
  asm volatile("" : "+v"(r0), "+v"(r1));
  return fmaxf(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1));
}
__device__ __forceinline__ float rows_max(float v) {
  const unsigned x = __builtin_bit_cast(unsigned, v);
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  const unsigned y = __builtin_bit_cast(unsigned, swap_max(a[0], a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(y, y, false, false);
  return swap_max(b[0], b[1]);
}

// Keys per pipeline tile and tiles in LDS (one multiplied, the rest in flight).
// Measured at batch 32 (per layer, fixed-chunk split): 64 x 2 stages 192 us,
// 32 x 3 200, 32 x 4 202, 32 x 5 205, 64 x 3 230 (96 KB: one workgroup per CU);
// balanced split (batch 32 / batch 8 x 32K / batch 64 x 4K): 64 x 2 169 / 221 /
// 302 us, 32 x 4 178 / 237 / 310, 32 x 3 (three workgroups per CU) 175 / 231 / 305.
constexpr int AT_KT = 64;
constexpr int AT_STG = 2;

// Keys [k_lo, k_hi) of one (sequence, kv head) for the wave's 16 query columns:
// the pipelined tile loop shared by both split kernels.  kt0 / vt0 point at the
// K / V fragments of key k_lo (a multiple of AT_KT); qload(qf) fills the wave's
// Q^T fragments while the first tiles are in flight.  Leaves the unnormalised
// output in oacc, the running max (log2 domain) in m_run and the sum of the
// probabilities, over the whole column, in l_run.
// qlim: the last key position this lane's query may see (causal passes; INT_MAX
// otherwise).  A lane all of whose keys lie past it leaves m_run = -inf, l_run = 0,
// which the merges skip.
// NT: stream the K / V tiles with the non-temporal cache policy.  Measured on the
// batch-32 ragged workload (balanced split, per layer): 145 us -> 123 us; a step of
// one 16-row block (fixed chunks, a few MB) is 0.3 us slower with it and keeps the
// default policy.
template <int D, int NW, int KT, int STG, bool NT, class QLoad>
__device__ __forceinline__ void attend_keys(f16x8* smem, const f16_t* kt0, const f16_t* vt0,
                                            int k_lo, int k_hi, QLoad qload, float& m_run,
                                            float& l_run, floatx4 (&oacc)[D / 16],
                                            int qlim = 0x7fffffff) {
  constexpr int NKT = KT / 16;             // 16-key blocks of a tile (S^T sub-tiles)
  constexpr int NH = KT / 32;              // 32-key blocks of a tile (V fragments' keys)
  constexpr int KFR = NKT * (D / 32);         // K fragments per tile
  constexpr int VFR = NH * (D / 16);          // V fragments per tile
  constexpr int TFR = KFR + VFR;
  constexpr int FPW = TFR / NW;               // fragments each wave loads per tile
  static_assert(TFR % NW == 0, "fragments per wave");
  static_assert(STG >= 2 && STG <= 5, "stages");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nt = (k_hi - k_lo + KT - 1) / KT;

  // tile i: K fragments from NKT i * D/32, V fragments from NH i * D/16
  auto issue = [&](int i) {
    f16x8* st = smem + (i % STG) * TFR * 64;
#pragma unroll
    for (int j = 0; j < FPW; ++j) {
      const int f = wave * FPW + j;
      const f16_t* g = f < KFR ? kt0 + ((long long)i * KFR + f) * 512
                               : vt0 + ((long long)i * VFR + f - KFR) * 512;
      if constexpr (NT)
        __builtin_amdgcn_global_load_lds((const void*)(g + lane * 8), (lds_void*)(st + f * 64), 16,
                                         0, AT_CPOL_NT);
      else
        __builtin_amdgcn_global_load_lds((const void*)(g + lane * 8), (lds_void*)(st + f * 64), 16,
                                         0, 0);
    }
  };
  for (int i = 0; i < STG - 1; ++i)
    if (i < nt) issue(i);

  // Q^T fragments already scaled by log2(e) / sqrt(d): the scores come out of the
  // products in the softmax's exp2 domain
  f16x8 qf[D / 32];
  qload(qf);

  m_run = -INFINITY;
  l_run = 0.f;
#pragma unroll
  for (int e = 0; e < D / 16; ++e) oacc[e] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int i = 0; i < nt; ++i) {
    // tile i has landed (the loads of the following tiles may still be in flight)
    vm_wait_tiles<FPW>(min(STG - 2, nt - 1 - i));
    barrier_pipelined();  // every wave's part of tile i is in LDS; tile i - 1 is no longer read
    if (i + STG - 1 < nt) issue(i + STG - 1);
    const int t0 = k_lo + i * KT;
    const int valid = min(KT, k_hi - t0);
    const f16x8* sK = smem + (i % STG) * TFR * 64;
    f16x8* sV = smem + (i % STG) * TFR * 64 + KFR * 64;
    if (valid < KT) {
      // last, partial tile: zero V at keys >= valid (stale cache contents; their
      // probabilities are 0 but 0 * inf would not be)
      for (int u = tid; u < VFR * 64; u += NW * 64) {
        const int h = (u / 64) / (D / 16), g = (u & 63) >> 4;
        f16x8 v = sV[u];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (32 * h + (j < 4 ? 4 * g + j : 16 + 4 * g + j - 4) >= valid) v[j] = (_Float16)0.f;
        sV[u] = v;
      }
      __syncthreads();
    }

    // S^T tile: NKT sub-tiles of 16 keys x 16 queries
    floatx4 sacc[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      sacc[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < D / 32; ++c)
        sacc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(sK[(kt * (D / 32) + c) * 64 + lane], qf[c],
                                                          sacc[kt], 0, 0, 0);
    }
    // mask (only a segment's partial last tile, or a causal pass's tile that reaches
    // past some lane's query; a wave-uniform test), tile max per query column
    float tmax = -INFINITY;
    if (valid < KT || __ballot(t0 + KT - 1 > qlim) != 0) {
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kt * 16 + (lane >> 4) * 4 + r;
          if (key >= valid || t0 + key > qlim) sacc[kt][r] = -INFINITY;
          tmax = fmaxf(tmax, sacc[kt][r]);
        }
    } else {
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, sacc[kt][r]);
    }
    tmax = rows_max(tmax);
    const float m_new = fmaxf(m_run, tmax);
    // no key of this lane seen yet (causal passes): every weight so far is 0
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float psum = 0.f;
    float pv[NH][8];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(sacc[kt][r] - m_use);
        psum += p;
        pv[kt >> 1][(kt & 1) * 4 + r] = p;
      }
    f16x8 pf[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) pf[h] = cvt8(pv[h]);
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int e = 0; e < D / 16; ++e) oacc[e] *= alpha;
    // O^T += V^T . P^T: V fragment (h, e) pairs with the probabilities of keys 32h..
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int e = 0; e < D / 16; ++e)
        oacc[e] = __builtin_amdgcn_mfma_f32_16x16x32_f16(sV[(h * (D / 16) + e) * 64 + lane], pf[h],
                                                         oacc[e], 0, 0, 0);
  }
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
}

// The lane's Q^T fragments: fp32 q times log2(e) / sqrt(d) (the score scale and the
// softmax's exp2 base, applied once per query instead of once per score), rounded to
// fp16; query row qrow, head hq, dims 32c + 8(lane/16)..; zero for lanes past the kv
// group's rows.
template <int D>
__device__ __forceinline__ void load_q(f16x8 (&qf)[D / 32], const float* q, int QD, bool qok,
                                       long long qrow, int hq) {
  const int lane = threadIdx.x & 63;
  const float sl2 = 1.4426950408889634f / sqrtf((float)D);
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    f16x8 h = {};
    if (qok) {
      const float* qp = q + qrow * QD + hq * D + c * 32 + (lane >> 4) * 8;
      h = cvt8(*(const floatx4*)qp * sl2, *(const floatx4*)(qp + 4) * sl2);
    }
    qf[c] = h;
  }
}

// Fixed-chunk split (one 16-row block step): grid (kv-head, split, sequence), kv
// heads fastest so the splits that hold keys (the first ones) are dispatched
// first and the empty ones after them;
// split s covers keys [s * chunk, (s + 1) * chunk) with chunk = fixed_chunk(keys of the
// sequence, n_split); splits past the end of a sequence have nothing to do (the merge
// skips them).  Partial slot (row, q-head, split): o[D], m, l, padding.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attn_split_mfma(DraftDims dd, const float* q,
                                                           const f16_t* kc, const f16_t* vc,
                                                           const int32_t* len, int n_split,
                                                           float* opart) {
  extern __shared__ f16x8 smem[];             // [AT_STG][tile fragments][64]: K, then V
  const int kvh = blockIdx.x, s = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = dd.Hq / dd.Hkv;
  const int B = dd.B;

  const int lb = len[b] + dd.pos_off;  // the block's first position
  int nk = lb + B;
  if (nk > dd.max_ctx) nk = dd.max_ctx;
  const int chunk = fixed_chunk(nk, n_split);
  const int k_lo = s * chunk;
  if (k_lo >= nk) return;
  const int k_hi = min(nk, k_lo + chunk);

  // query handled by this lane (column of S^T): group row qr = 16*wave + lane%16
  const int qr = wave * 16 + (lane & 15);
  const bool qok = qr < G * B;
  const int hq = kvh * G + (qok ? qr / B : 0);
  const int rr = qok ? qr % B : 0;
  const long long qrow = (long long)b * B + rr;
  const int qlim = dd.causal ? lb + rr : 0x7fffffff;

  const long long slice = ((long long)b * dd.Hkv + kvh) * dd.max_ctx * D;
  const f16_t* kt0 = kc + slice + (long long)(k_lo >> 4) * (D / 32) * 512;
  const f16_t* vt0 = vc + slice + (long long)(k_lo >> 5) * (D / 16) * 512;
  float m_run, l_run;
  floatx4 oacc[D / 16];
  attend_keys<D, NW, AT_KT, AT_STG, false>(smem, kt0, vt0, k_lo, k_hi,
                     [&](f16x8(&qf)[D / 32]) { load_q<D>(qf, q, dd.Hq * D, qok, qrow, hq); },
                     m_run, l_run, oacc, qlim);

  constexpr int SP = D + 32;  // partial slot pitch: o[D], m, l, padding
  if (qok) {
    const long long slot = ((qrow * dd.Hq + hq) * n_split + s);
    float* op = opart + slot * SP;
#pragma unroll
    for (int e = 0; e < D / 16; ++e)
#pragma unroll
      for (int r = 0; r < 4; ++r) op[e * 16 + (lane >> 4) * 4 + r] = oacc[e][r];
    if ((lane >> 4) == 0) {
      op[D] = m_run;
      op[D + 1] = l_run;
    }
  }
}

// ---- work-balanced split (batched steps) ------------------------------------------------
// The keys of every (sequence b, kv head h) segment, in 64-key tiles, are laid
// end to end in the order (b, h, tile), each segment led by AT_PIECE_COST virtual
// tiles that stand for what starting a piece costs (loading Q, the pipeline's first
// tile, the partial's stores): segment g = b * Hkv + h spans flattened tiles
// [Hkv * C_b + h * v_b, + v_b) with v_b = n_b + AT_PIECE_COST, n_b = ceil(min(len_b + B,
// max_ctx) / 64) real tiles and C_b = v_0 + .. + v_{b-1}; V tiles in all.  Workgroup w of
// P takes flattened tiles [floor(w V / P), floor((w + 1) V / P)) (P at most V), so every
// workgroup gets the same cost whatever the mix of context lengths: one that starts
// more pieces streams fewer tiles.  The real tiles of a segment a workgroup covers
// are one piece (none when its share holds only virtual ones): its partial (o, m, l)
// per query row goes to slot w + g, which is unique because along the flattened
// order each next piece advances w, g or both (at most P + segments slots).  The
// workgroup that holds a segment's first real tile records (w, pieces of the
// segment) in meta[g] for the merge.
__device__ __forceinline__ int seq_keys(const int32_t* len, int b, const DraftDims& dd) {
  int nk = len[b] + dd.pos_off + dd.B;
  if (nk > dd.max_ctx) nk = dd.max_ctx;
  return nk < 1 ? 1 : nk;
}
__device__ __forceinline__ int seq_keys_uniform(const int32_t* len, int b, const DraftDims& dd) {
  return __builtin_amdgcn_readfirstlane(seq_keys(len, __builtin_amdgcn_readfirstlane(b), dd));
}

__device__ __forceinline__ long long uniform64(long long v) {
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)(unsigned long long)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)((unsigned long long)v >> 32));
  return (long long)(((unsigned long long)hi << 32) | lo);
}

// wave-wide inclusive prefix sum over 64 lanes
__device__ __forceinline__ long long wave_incl_scan(long long v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const long long u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  return v;
}

// Total flattened tiles over all sequences (per kv head; `lead` virtual tiles lead
// each segment), and the sequence b holding per-head-scaled flattened tile t
// (Hkv C_b <= t < Hkv C_{b+1}) with C_b and v_b; one wave-wide scan per 64
// sequences; every wave computes the same.
__device__ __forceinline__ long long total_seq_tiles(const int32_t* len, const DraftDims& dd,
                                                     int kt, int lead) {
  const int lane = threadIdx.x & 63;
  long long tot = 0;
  for (int c0 = 0; c0 < dd.batch; c0 += 64) {
    const int bb = c0 + lane;
    long long my = bb < dd.batch ? (seq_keys(len, bb, dd) + kt - 1) / kt + lead : 0;
    tot += __shfl(wave_incl_scan(my), 63, 64);
  }
  return uniform64(tot);
}

__device__ __forceinline__ void locate_seq(const int32_t* len, const DraftDims& dd, int kt,
                                           int lead, long long t, int& b, long long& cb,
                                           int& nb) {
  const int lane = threadIdx.x & 63;
  long long carry = 0;
  for (int c0 = 0; c0 < dd.batch; c0 += 64) {
    const int bb = c0 + lane;
    const long long my = bb < dd.batch ? (seq_keys(len, bb, dd) + kt - 1) / kt + lead : 0;
    const long long incl = wave_incl_scan(my);
    // sequences of this chunk that end at or before t
    const unsigned long long before = __ballot((long long)dd.Hkv * (carry + incl) <= t);
    const int cnt = __popcll(before);
    if (cnt < 64 && c0 + cnt < dd.batch) {
      b = c0 + cnt;
      cb = uniform64(carry + __shfl(incl - my, cnt, 64));
      nb = __builtin_amdgcn_readfirstlane((int)__shfl(my, cnt, 64));
      return;
    }
    carry += uniform64(__shfl(incl, 63, 64));
  }
  b = dd.batch - 1;  // not reached for t < Hkv * total
  cb = carry;
  nb = 1;
}

template <int D, int NW, int KT, int STG>
__global__ __launch_bounds__(NW * 64) void attn_lean_mfma(DraftDims dd, const float* q,
                                                          const f16_t* kc, const f16_t* vc,
                                                          const int32_t* len, float* opart,
                                                          int32_t* meta) {
  extern __shared__ f16x8 smem[];
  const int w = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = dd.Hq / dd.Hkv, B = dd.B, GB = G * B, Hkv = dd.Hkv;
  constexpr int SP = D + 4;  // partial slot pitch: o[D], m, l, padding to 16 bytes

  constexpr int LEAD = AT_PIECE_COST;
  const long long V = (long long)Hkv * total_seq_tiles(len, dd, KT, LEAD);
  // no more workgroups than flattened tiles, so the workgroups of a segment are
  // consecutive
  const int P = (int)min((long long)gridDim.x, V);
  if (w >= P) return;
  const long long lo = (long long)w * V / P;
  const long long hi = (long long)(w + 1) * V / P;
  if (lo >= hi) return;
  int b, vb;
  long long cb;
  locate_seq(len, dd, KT, LEAD, lo, b, cb, vb);
  int kvh = (int)((lo - (long long)Hkv * cb) / vb);
  long long tg = (long long)Hkv * cb + (long long)kvh * vb;  // segment's first flattened tile
  int nk = seq_keys_uniform(len, b, dd);

  const int qr = wave * 16 + (lane & 15);
  const bool qok = qr < GB;
  for (bool first = true;;) {
    // this workgroup's real tiles of the segment at tg: flattened [rs, re)
    const long long rs = max(lo, tg + LEAD), re = min(hi, tg + vb);
    if (rs < re) {
      const int off = (int)(rs - tg - LEAD), n = (int)(re - rs);
      const int k_lo = off * KT, k_hi = min(nk, (off + n) * KT);
      const int g = b * Hkv + kvh;
      if (off == 0 && threadIdx.x == 0) {
        // the last real tile's workgroup: min(P - 1, ceil((t + 1) P / V) - 1)
        const long long tl = tg + vb - 1;
        const long long wl = min((long long)P - 1, ((tl + 1) * P - 1) / V);
        meta[2 * g] = w;
        meta[2 * g + 1] = (int)(wl - w + 1);
      }
      if (!first) {
        vm_wait_tiles<1>(0);  // the previous piece's partial stores are out of the wait counts
        __syncthreads();      // and its last tile is no longer read
      }
      first = false;

      const int hq = kvh * G + (qok ? qr / B : 0);
      const long long qrow = (long long)b * B + (qok ? qr % B : 0);
      const long long slice = ((long long)b * Hkv + kvh) * dd.max_ctx * D;
      const f16_t* kt0 = kc + slice + (long long)(k_lo >> 4) * (D / 32) * 512;
      const f16_t* vt0 = vc + slice + (long long)(k_lo >> 5) * (D / 16) * 512;
      const int qlim = dd.causal ? len[b] + dd.pos_off + (qok ? qr % B : 0) : 0x7fffffff;
      float m_run, l_run;
      floatx4 oacc[D / 16];
      attend_keys<D, NW, KT, STG, true>(smem, kt0, vt0, k_lo, k_hi,
                         [&](f16x8(&qf)[D / 32]) { load_q<D>(qf, q, dd.Hq * D, qok, qrow, hq); },
                         m_run, l_run, oacc, qlim);
      if (qok) {
        float* op = opart + ((long long)(w + g) * GB + qr) * SP;
#pragma unroll
        for (int e = 0; e < D / 16; ++e) *(floatx4*)(op + e * 16 + (lane >> 4) * 4) = oacc[e];
        if ((lane >> 4) == 0) {
          op[D] = m_run;
          op[D + 1] = l_run;
        }
      }
    }
    if (tg + vb >= hi) break;
    // the next segment: the next kv head of this sequence, or the next sequence
    tg += vb;
    if (++kvh == Hkv) {
      kvh = 0;
      ++b;
      nk = seq_keys_uniform(len, b, dd);
      vb = (nk + KT - 1) / KT + LEAD;
    }
  }
}

// log-sum-exp merge of a segment's pieces: D/4 lanes per (row, q-head), four
// dims each, so a wave merges 128 / D * 2 of them; the pieces' slots follow
// from meta (two memory latencies); pieces are read four at a time and folded
// in with a running maximum.  No LDS, no barriers.
template <int D>
__global__ __launch_bounds__(256) void attn_lean_merge(DraftDims dd, const int32_t* meta,
                                                        const float* opart, float* o,
                                                        uint16_t* opack, int npairs) {
  constexpr int SP = D + 4;
  constexpr int LPP = D / 4;    // lanes per (row, q-head)
  constexpr int PPW = 64 / LPP;  // (row, q-head) pairs per wave
  const int lane = threadIdx.x & 63;
  const int pair = (blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) * PPW + lane / LPP;
  if (pair >= npairs) return;
  const int e = (lane % LPP) * 4;
  const int qrow = pair / dd.Hq, hq = pair % dd.Hq;
  const int G = dd.Hq / dd.Hkv, GB = G * dd.B;
  const int b = qrow / dd.B, r = qrow % dd.B, kvh = hq / G;
  const int g = b * dd.Hkv + kvh, qr = (hq % G) * dd.B + r;
  const int w0 = meta[2 * g], np = meta[2 * g + 1];
  const float* base = opart + ((long long)(w0 + g) * GB + qr) * SP;
  const long long pitch = (long long)GB * SP;  // from one piece's row to the next's
  float m = -INFINITY, l = 0.f;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < np; s0 += 4) {
    float2 ml[4];
    floatx4 ov[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float* pp = base + min(s0 + j, np - 1) * pitch;
      ml[j] = *(const float2*)(pp + D);
      ov[j] = *(const floatx4*)(pp + e);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (s0 + j < np && ml[j].y > 0.f) {
        const float mn = fmaxf(m, ml[j].x);
        const float a = exp2f(m - mn), c = exp2f(ml[j].x - mn);
        acc = acc * a + ov[j] * c;
        l = l * a + ml[j].y * c;
        m = mn;
      }
  }
  const floatx4 v = acc / l;
  if (opack) {
    const int k = hq * D + e, KT = dd.Hq * D / 32;
    const long long idx =
        (((long long)(qrow >> 4) * KT + (k >> 5)) * 64 + (qrow & 15) + 16 * ((k & 31) >> 3)) * 8 + (k & 7);
    uint2 pk;
    pk.x = (uint32_t)f2h(v[0]) | ((uint32_t)f2h(v[1]) << 16);
    pk.y = (uint32_t)f2h(v[2]) | ((uint32_t)f2h(v[3]) << 16);
    *(uint2*)(opack + idx) = pk;
  } else {
    *(floatx4*)(o + (long long)qrow * dd.Hq * D + hq * D + e) = v;
  }
}

// log-sum-exp merge of the active splits of a row's sequence: one workgroup per
// (row, q-head), one thread per dim.  Two memory latencies: the sequence length,
// every split's (m, l) and every dim's partial of the first AT_MERGE_PRE splits
// are requested together (clamped to existing slots; values of inactive splits
// are ignored), and only partials of splits beyond those are fetched after.
constexpr int AT_MERGE_PRE = 32;
// o: fp32 rows [M][Hq * D], or (opack non-null) fp16 fragments in the packed A
// layout of the output projection (K = Hq * D, rows padded to 256).
template <int D>
__global__ __launch_bounds__(D) void attn_merge(DraftDims dd, int n_split, const int32_t* len,
                                                 const float* opart, float* o, uint16_t* opack) {
  constexpr int SP = D + 32;
  constexpr int SPT = AT_MAX_SPLIT / D;  // splits per thread for the weights
  __shared__ float sw[AT_MAX_SPLIT];
  __shared__ float red[2][D / 64];
  const int qrow = blockIdx.x, hq = blockIdx.y, e = threadIdx.x;
  const float* op = opart + ((long long)qrow * dd.Hq + hq) * n_split * SP;
  int nk = len[qrow / dd.B] + dd.pos_off + dd.B;
  float ms[SPT], ls[SPT];
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const int s = min(e + j * D, n_split - 1);
    ms[j] = op[s * SP + D];
    ls[j] = op[s * SP + D + 1];
  }
  float t[AT_MERGE_PRE];
#pragma unroll
  for (int s = 0; s < AT_MERGE_PRE; ++s) t[s] = op[min(s, n_split - 1) * SP + e];
  if (nk > dd.max_ctx) nk = dd.max_ctx;
  const int chunk = fixed_chunk(nk, n_split);
  const int na = min(n_split, (nk + chunk - 1) / chunk);  // splits that wrote a partial
  // split weights w_s = exp2(m_s - max m) (0 for empty splits), L = sum w_s l_s
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < SPT; ++j)
    if (e + j * D < na && ls[j] > 0.f) mx = fmaxf(mx, ms[j]);
  mx = warp_max(mx);
  if ((e & 63) == 0) red[0][e >> 6] = mx;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < D / 64; ++w) mx = fmaxf(mx, red[0][w]);
  float L = 0.f;
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const int s = e + j * D;
    const bool act = s < na && ls[j] > 0.f;  // slots past na hold whatever an earlier call left
    const float w = act ? exp2f(ms[j] - mx) : 0.f;
    if (s < na) sw[s] = w;
    if (act) L += w * ls[j];  // never 0 * (a stale NaN or infinity)
  }
  L = warp_sum(L);
  if ((e & 63) == 0) red[1][e >> 6] = L;
  __syncthreads();  // sw and the partial L sums are visible
  float Lt = 0.f;
#pragma unroll
  for (int w = 0; w < D / 64; ++w) Lt += red[1][w];
  float acc = 0.f;
#pragma unroll
  for (int s = 0; s < AT_MERGE_PRE; ++s)
    if (s < na) acc += sw[s] * t[s];
  for (int s0 = AT_MERGE_PRE; s0 < na; s0 += 8) {  // loads issued 8 at a time, summed in order
    float u[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) u[j] = op[min(s0 + j, na - 1) * SP + e];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + j < na) acc += sw[s0 + j] * u[j];
  }
  const float v = acc / Lt;
  if (opack) {
    const int k = hq * D + e, KT = dd.Hq * D / 32;
    opack[(((long long)(qrow >> 4) * KT + (k >> 5)) * 64 + (qrow & 15) + 16 * ((k & 31) >> 3)) * 8 +
          (k & 7)] = f2h(v);
  } else {
    o[(long long)qrow * dd.Hq * D + hq * D + e] = v;
  }
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
  int nk = len[b] + dd.pos_off + dd.B;
  if (dd.causal) nk = len[b] + dd.pos_off + r + 1;  // keys up to the row's own position
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

// Splits of the fixed-chunk attention (the grid's split dimension): no more than the
// 64-key tiles of max_ctx.
int attention_splits(const DraftDims& dd) {
  return (int)std::min<long long>(AT_FIXED_SPLITS, (dd.max_ctx + AT_CHUNK_UNIT - 1) / AT_CHUNK_UNIT);
}

// A step of one 16-row block keeps the fixed-chunk split (up to AT_FIXED_SPLITS
// workgroups per (sequence, kv head), a one-latency merge); batched steps use the
// balanced split.
static bool attention_balanced(const DraftDims& dd) { return dd.batch * dd.B > 16; }

// Workgroups of the balanced split: every CU holds two (their LDS fits one CU),
// all resident at once; no more than there are tiles.  Measured per layer
// (batch 32 ragged / batch 8 x 32K / batch 64 x 4K): 256 -> 201 / 227 / 399 us,
// 512 -> 188 / 219 / 346, 768 and 1024 slower again.
constexpr int AT_LEAN_GRID = 512;
static int attention_lean_grid(const DraftDims& dd) {
  const long long tiles = (long long)dd.batch * dd.Hkv * (dd.max_ctx / AT_KT);
  return (int)(tiles < AT_LEAN_GRID ? tiles : AT_LEAN_GRID);
}

size_t attention_part_bytes(int dtype, const DraftDims& dd) {
  if (dtype == 0) return 0;
  // fixed chunks: room for attention_splits(dd) splits, which never decreases as
  // max_ctx grows
  if (!attention_balanced(dd))
    return (size_t)dd.batch * dd.B * dd.Hq * attention_splits(dd) * (dd.d + 32) * 4;
  const size_t segs = (size_t)dd.batch * dd.Hkv;
  const size_t slots = (size_t)attention_lean_grid(dd) + segs;
  return (slots * (dd.Hq / dd.Hkv) * dd.B * (dd.d + 4) + 2 * segs) * 4;
}

template <int D, int NW, int KT, int STG>
static hipError_t launch_lean(const DraftDims& dd, int P, const float* q, const void* kc,
                              const void* vc, const int32_t* len, float* opart, int32_t* meta,
                              hipStream_t st, LaunchEvents ev) {
  const size_t lds = (size_t)STG * (KT / 16 * (D / 32) + KT / 32 * (D / 16)) * 1024;
  const hipError_t e = set_lds_limit((const void*)attn_lean_mfma<D, NW, KT, STG>, (int)lds);
  if (e != hipSuccess) return e;
  DF_LAUNCH(ev.start, ev.stop, (attn_lean_mfma<D, NW, KT, STG>), P, NW * 64, lds, st, dd, q,
            (const f16_t*)kc, (const f16_t*)vc, len, opart, meta);
  return hipSuccess;
}

hipError_t launch_attention(int dtype, const DraftDims& dd, const float* q, const void* kc,
                            const void* vc, const int32_t* len, float* opart, float* o,
                            hipStream_t st, LaunchEvents ev, uint16_t* opack) {
  if (dtype == 0) {
    if (dd.d > 128) return hipErrorInvalidValue;
    dim3 grid(dd.B, dd.Hq, dd.batch);
    DF_LAUNCH(ev.start, ev.stop, attn_f32, grid, 128, 0, st, dd, q, (const float*)kc, (const float*)vc,
              len, o);
    return hipGetLastError();
  }
  const int G = dd.Hq / dd.Hkv;
  const int rows = G * dd.B;  // query rows of a kv group: one wave per 16, 4 or 8 waves
  if (rows > 128) return hipErrorInvalidValue;
  if (dd.max_ctx % AT_CHUNK_UNIT) return hipErrorInvalidValue;
  const bool lean = attention_balanced(dd);
  const int n_split = attention_splits(dd);
  if (!lean && n_split > AT_MAX_SPLIT) return hipErrorInvalidValue;
  const int P = attention_lean_grid(dd);
  int32_t* meta = (int32_t*)(opart + (size_t)(P + dd.batch * dd.Hkv) * rows * (dd.d + 4));
  dim3 grid(dd.Hkv, n_split, dd.batch);
  dim3 mgrid(dd.batch * dd.B, dd.Hq);
  const int npairs = dd.batch * dd.B * dd.Hq;             // (row, q-head) pairs to merge
  const int lgrid = (npairs + 4 * (256 / dd.d) - 1) / (4 * (256 / dd.d));  // 4 waves of 128/d*2
  hipEvent_t none = nullptr;
  const size_t lds = (size_t)AT_STG * (AT_KT / 16 * (dd.d / 32) + AT_KT / 32 * (dd.d / 16)) * 1024;
#define AT_ATTR(K)                                                                               \
  {                                                                                              \
    const hipError_t e = set_lds_limit((const void*)K, (int)lds);                                \
    if (e != hipSuccess) return e;                                                               \
  }
#define AT_LAUNCH(D, NW)                                                                          \
  if (lean) {                                                                                    \
    hipError_t le = launch_lean<D, NW, AT_KT, AT_STG>(dd, P, q, kc, vc, len, opart, meta, st,   \
                                                      ev);                                       \
    if (le != hipSuccess) return le;                                                             \
    DF_LAUNCH(none, none, attn_lean_merge<D>, lgrid, 256, 0, st, dd, (const int32_t*)meta,       \
              (const float*)opart, o, opack, npairs);                                            \
  } else {                                                                                       \
    AT_ATTR((attn_split_mfma<D, NW>))                                                            \
    DF_LAUNCH(ev.start, ev.stop, (attn_split_mfma<D, NW>), grid, NW * 64, lds, st, dd, q,       \
              (const f16_t*)kc, (const f16_t*)vc, len, n_split, opart);                         \
    DF_LAUNCH(none, none, attn_merge<D>, mgrid, D, 0, st, dd, n_split, len, opart, o,             \
              opack);                                                                           \
  }
  if (dd.d == 128) {
    if (rows <= 64) {
      AT_LAUNCH(128, 4)
    } else {
      AT_LAUNCH(128, 8)
    }
  } else if (dd.d == 64) {
    if (rows <= 64) {
      AT_LAUNCH(64, 4)
    } else {
      AT_LAUNCH(64, 8)
    }
  } else {
    return hipErrorInvalidValue;
  }
#undef AT_ATTR
#undef AT_LAUNCH
  return hipGetLastError();
}
