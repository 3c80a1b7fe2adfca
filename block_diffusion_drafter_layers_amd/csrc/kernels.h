// Internal launchers of the DFlash kernels (host side).  Not part of the C ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

// Optional timing of one launch: events recorded by the dispatch itself at the
// kernel's start and end (hipExtLaunchKernel), so they bracket the kernel and
// nothing else.  Both null: a plain launch.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  bool on() const { return start || stop; }
};

// kernel<<<grid, block, lds, st>>>(args...), or the event-recording launch
#define DF_LAUNCH(ev_start, ev_stop, kernel, grid, block, lds, st, ...)                          \
  do {                                                                                          \
    if ((ev_start) || (ev_stop))                                                                \
      hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(block), (uint32_t)(lds), st, ev_start,    \
                            ev_stop, 0, __VA_ARGS__);                                          \
    else                                                                                        \
      kernel<<<grid, block, lds, st>>>(__VA_ARGS__);                                            \
  } while (0)

#define DF_MAX_ASEG 8
#define DF_MAX_WSEG 64
#define DF_MAX_LAYERS 32

struct LayerPtrs {
  void* k[DF_MAX_LAYERS];
  void* v[DF_MAX_LAYERS];
};

// fuse_inject's row map (packed row -> sequence, cache position), computed by a
// kernel that owns rows row0.. of the call: seq/pos indexed by the kernel's row.
struct RowMap {
  int batch, max_ctx, row0;
  const int32_t *row_start, *row_count, *len;
  int32_t *seq, *pos, *err;
};

// Advance of len at the end of a fuse_inject call (after the row map has read it).
struct LenUpdate {
  int batch, total_rows, max_ctx;
  const int32_t *row_start, *row_count;
  int32_t *len, *err;
};

// Row statistics for RMSNorm travel as partial sums of squares, one per
// SS_COLS-column chunk (the 16 columns of one matrix-core output group, so a
// kernel that owns only some 16-column groups of a row can still write them):
// ss[m * ss_chunks(N) + c].
#define SS_COLS 16
__host__ __device__ inline int ss_chunks(int n) { return (n + SS_COLS - 1) / SS_COLS; }

// out[s][m][n] = sum_{k in split s} A[m, k] * W[n, k]   (fp32 partial sums)
//   A[m, k] = a[k / ka_w][m * lda + k % ka_w]      (K split into equal-width pointer segments)
//   W[n, k] = segment j (n_off[j] <= n < n_off[j+1]), row n - n_off[j]: fp32 row-major
//             with row pitch ldw, or fp16 fragment-packed with K columns (launch_pack_weight);
//             packed segment boundaries are multiples of 16
struct GemmArgs {
  int M, N, K;
  int S, kc;  // number of K splits and K extent of each (filled by plan_gemm)
  int kind;   // GEMM_* (filled by plan_gemm)
  int a_f32;  // 1: A is an fp32 activation; 0: A has the storage type (bf16 features)
  int n_aseg, ka_w;
  long long lda, ldw;
  const void* a[DF_MAX_ASEG];
  int n_wseg;
  const void* w[DF_MAX_WSEG];
  int n_off[DF_MAX_WSEG + 1];
  float* out;
  // optional RMSNorm of the A rows folded into the staging of A (fp32 A only):
  // A[m, k] <- A[m, k] * rsqrt(sum_c nss[m * nss_chunks + c] / K + neps) * ngain[k]
  const float* nss;
  int nss_chunks;
  const void* ngain;  // weights' type
  float neps;
  int wps, grid;      // skinny: workgroups per K split (each loops over tiles); grid = S * wps
  uint16_t* apack;    // mfma: workspace for the packed fp16 A rows (gemm_apack_bytes)
  // mfma, one K split, two weight segments (gate, up) of I = N / 2 rows each,
  // I % 128 == 0: the output is silu(gate) * up, written to swiglu_out as fp16
  // fragments in the packed A layout of a GEMM with K = I (rows padded to 256;
  // out is not written)
  uint16_t* swiglu_out;
  // mfma: apack already holds A in the packed layout (no packing pass)
  int a_packed;
  // mfma: output tile, 256 (256 x 256) or 128 (128 x 128), filled by plan_gemm;
  // 384 (128 x 384, SwiGLU epilogue only), set by plan_swiglu
  int tile;
};

enum { GEMM_F32 = 0, GEMM_SKINNY1 = 1, GEMM_SKINNY2 = 2, GEMM_SKINNY4 = 3, GEMM_MFMA = 4 };

// Choose the kernel and the split of K for a shape; returns S.
int plan_gemm(GemmArgs& g, int dtype);
// After plan_gemm, for a gate|up GEMM (two weight segments of I = N / 2 rows): true
// when the SwiGLU epilogue fits the plan (matrix cores, one K split, I % 128 == 0),
// then with the tile that fills the CUs best (256 x 256, or 128 x 384 when
// I % 192 == 0 and it takes fewer tile-rounds).  The caller then sets swiglu_out.
bool plan_swiglu(GemmArgs& g);
// Workspace the planned GEMM needs for its packed A rows (0 unless GEMM_MFMA).
size_t gemm_apack_bytes(const GemmArgs& g);
hipError_t launch_gemm(const GemmArgs& g, int dtype, hipStream_t st, LaunchEvents ev = {});
// Full-K GEMMs for M <= 16 rows (bf16 storage, packed fp16 weights [N][K], A one
// 16-row group of packed fp16 fragments).  No partial sums, no reduce kernel.
//   resid:    X[m][n] += sum_k A[m][k] W[n][k]; ss_out = 16-column chunk statistics of the new X
//   resid_y:  as resid, and y = the next GEMM's packed A rows fp16(X_new * gain * sc[m]) with
//             sc[m] = rsqrt(mean(X_old^2) + eps) from ss_in (statistics of X before the
//             update; ss_in != ss_out), sc written (16 floats)
//   swiglu:   A as written by resid_y (K = hidden); r = rsqrt(mean(X^2) + eps) / sc from
//             ss_in (statistics of that X); out = packed silu(r A Wg^T) * (r A Wu^T), I columns
//   qkv:      A as for swiglu; Q | K | V with RoPE (the rope table of launch_embed): q rows
//             [M][Hq d] and the block's K/V rows in this layer's packed fp16 cache at
//             positions len[b] + j (row m = b B + j; positions >= max_ctx are not written)
bool rowk_fits(int M, int N, int K, bool gate_up);
bool rowk_qkv_fits(int M, int K, int d);
hipError_t launch_rowk_qkv(const void* A, const void* Wq, const void* Wk, const void* Wv, int M,
                           int K, int B, int Hq, int Hkv, int d, const float* ss_in, float eps,
                           const float* sc, const int32_t* len, const float* rope, float* q,
                           void* kc, void* vc, int max_ctx, hipStream_t st, LaunchEvents ev = {});
hipError_t launch_rowk_resid(const void* A, const void* W, int M, int N, int K, float* X,
                             float* ss_out, hipStream_t st, LaunchEvents ev = {});
hipError_t launch_rowk_resid_y(const void* A, const void* W, int M, int N, int K, float* X,
                               float* ss_out, const float* ss_in, const void* gain, float eps,
                               float* sc, void* y, hipStream_t st, LaunchEvents ev = {});
hipError_t launch_rowk_swiglu(const void* A, const void* Wg, const void* Wu, int M, int I, int K,
                              const float* ss_in, float eps, const float* sc, void* out,
                              hipStream_t st, LaunchEvents ev = {});
// bf16 W[N][K] row-major -> fragment-packed fp16 (N % 16 == 0, K % 32 == 0; no overlap);
// elements that do not fit fp16 are added to *n_overflow (nullable).
hipError_t launch_pack_weight(const void* src, int N, int K, void* dst, int32_t* n_overflow,
                              hipStream_t st);

// ---- elementwise / normalisation / attention / head ----------------------------
struct DraftDims {
  int H, Hq, Hkv, d, I, V, B, batch, max_ctx, mask_id;
  float theta, eps;
  // the block's rows sit at positions len[b] + pos_off + r (0 for a draft)
  int pos_off = 0;
  // 1: block row r sees keys up to position len[b] + pos_off + r only (the
  // autoregressive passes of the target and of the input-fusion injection);
  // 0: every key (the drafter's non-causal block)
  int causal = 0;
};

// Activations exchanged between kernels are fp32.  `dtype` is the storage type:
// fp32 -> fp32 weights, cache and lm_head rows; bf16 -> bf16 gains and
// embedding, fp16 packed matrices, fp16 cache and lm_head rows.

// X[m] = embed[id(m)] (id = last_tok[b] for block row 0, mask id otherwise) and
// its ss partials; RoPE cos/sin of positions len[b] + r into rope[m][d/2][2];
// base[b] = len[b]; overflow / token range errors.
hipError_t launch_embed(int dtype, const DraftDims& dd, const int32_t* last_tok, const void* embed,
                        int32_t* len, int32_t* base, int32_t* err, float* X, float* ss,
                        float* rope, hipStream_t st, const void* gain = nullptr,
                        float* sc = nullptr, void* y = nullptr, const int32_t* ids = nullptr);
// (ids non-null: row m embeds token ids[m], a block of given tokens)
// Rows of a causal pass fed with fused features (input-fusion injection): block row
// m = b B + j takes packed row row_start[b] + pos_off + j of y, RMS-normalised with
// its ss partials y_ss and the gain, or zero past row_count[b]; its ss partials and
// RoPE table at position len[b] + pos_off + j.
hipError_t launch_gather_rows(int dtype, const DraftDims& dd, const float* y, const float* y_ss,
                              const void* gain, const int32_t* row_start,
                              const int32_t* row_count, const int32_t* len, float* X, float* ss,
                              float* rope, hipStream_t st);
// len[b] += add (clamped to max_ctx, overflow bit)
hipError_t launch_len_add(int batch, int add, int32_t* len, int max_ctx, int32_t* err,
                          hipStream_t st);
// out = X [M][H] fp32 in the storage type (bf16 or fp32)
hipError_t launch_store_rows(int dtype, int M, int H, const float* X, void* out, hipStream_t st);
// (y non-null: one 16-row group, bf16; also y = packed fp16 RMSNorm(X) * gain rows and
// sc[m] = rsqrt(mean(X^2) + eps), the scale y carries)
// out[m, n] = (accumulate ? out[m, n] : 0) + sum_s P[s][m][n]; ss partials of the new rows;
// with rm non-null also fuse_inject's row map of its rows.
hipError_t launch_reduce_rows(int M, int N, const float* P, int S, float* out, bool accumulate,
                              float* ss, hipStream_t st,
                              const RowMap* rm = nullptr);
// Batched path (bf16 storage, N % 256 == 0): as launch_reduce_rows with one
// workgroup per row; with apack non-null also the new rows RMS-normalised by
// gain (bf16) as fp16 packed A rows of the next GEMM (K = N; rows >= M untouched);
// with rm non-null also fuse_inject's row map of its rows.
hipError_t launch_reduce_pack(int M, int N, const float* P, int S, float* out, bool accumulate,
                              float* ss, const void* gain, float eps, void* apack,
                              hipStream_t st, const RowMap* rm = nullptr);
// y = src * rsqrt(mean(src^2) + eps) * gain from the ss partials.  z (weights' type,
// nullable) receives rows with (row % compact_B) != 0 packed (compact_B = 0: all rows);
// dbg (fp32, nullable) receives every row.
hipError_t launch_norm_rows(int dtype, int M, int N, const float* src, const float* ss,
                            int ss_nch, const void* gain, float eps, void* z, int compact_B,
                            float* dbg, hipStream_t st);
hipError_t launch_qkv_post(int dtype, const DraftDims& dd, const float* P, int S,
                           const int32_t* len, const float* rope, float* q, void* kc, void* vc,
                           hipStream_t st);
// pout non-null: the result as packed fp16 A rows (K = I, rows padded to 16) instead of fp32 rows
hipError_t launch_swiglu(int M, int I, const float* P, int S, float* out, hipStream_t st,
                         uint16_t* pout = nullptr);
// Split-K attention (bf16 weights) followed by the log-sum-exp merge of the splits.
// kc/vc: the layer's cache, fp32 (fp32 storage type) or fp16 (bf16 storage type).
// opack (bf16 storage only, nullable): o is written as packed fp16 A rows of the
// output projection instead of fp32 rows.
// opart: attention_part_bytes(dtype, dd) of workspace (split partials and, for
// batched steps, the balanced split's piece table).
hipError_t launch_attention(int dtype, const DraftDims& dd, const float* q, const void* kc,
                            const void* vc, const int32_t* len, float* opart, float* o,
                            hipStream_t st, LaunchEvents ev = {}, uint16_t* opack = nullptr);
size_t attention_part_bytes(int dtype, const DraftDims& dd);
// kcs/vcs: host arrays of n_layers device pointers.  With len non-null the same
// launch also does launch_len_update's work (the call's last pass).
hipError_t launch_inject_post(int dtype, int rows, int n_layers, int Hkv, int d, int max_ctx,
                              float theta, const float* P, int S, const int32_t* seq,
                              const int32_t* pos, void* const* kcs, void* const* vcs,
                              hipStream_t st, int batch = 0, int total_rows = 0,
                              const int32_t* row_start = nullptr,
                              const int32_t* row_count = nullptr, int32_t* len = nullptr,
                              int32_t* err = nullptr);
hipError_t launch_len_update(int batch, int total_rows, const int32_t* row_start,
                             const int32_t* row_count, int32_t* len, int max_ctx, int32_t* err,
                             hipStream_t st);
hipError_t launch_accept_trim(int batch, int B, const int32_t* drafts, const int32_t* targets,
                              int32_t* accept_len, int32_t* bonus, int32_t* len,
                              const int32_t* base, int32_t* err, hipStream_t st);
// Gumbel-max sampling of the drafted tokens: a row's pick becomes
// argmax_v(logit_v / T + g_v) with standard Gumbel noise g_v = -log(-log u_v),
// u_v = (2 floor(x / 2^9) + 1) / 2^24 from word x = (v / 16) % 4 of the
// Philox4x32-10 block at counter (v with bits 4 and 5 cleared, position,
// sequence, offset) and key (k0, k1) = the seed's low and high halves (one block
// serves ids v, v+16, v+32, v+48, which one lane of the batched head holds); the position of
// kernel row m (rows 1..B-1 of each block, in order) is base[b] + m % (B-1) + 1
// with b = m / (B-1).  inv_t = 0: the plain argmax.
struct DraftSampler {
  float inv_t = 0.f;
  uint32_t k0 = 0, k1 = 0, offset = 0;
  const int32_t* base = nullptr;
  int rows_per_seq = 1;
};

// lm_head + argmax over rows Z [R, H]; partial results then reduced into ids.
// Partial tiles of the variant that serves (R, with_logits, top2); top2: the
// runner-up is tracked too (fp32 kernel, or the 128-wide tiles).
int lmhead_tiles(int dtype, int R, int V, int H, bool with_logits, bool top2 = false);
// The 16-row group head (launch_lmhead_group) serves R rows of hidden size H.
bool lmhead_group_fits(int R, int H);
// bf16 storage, R > 16 rows: Zp holds the rows packed (launch_norm_pack), padded to 256.
hipError_t launch_lmhead_packed(int R, int V, int H, const void* Zp, const void* W, float* pval,
                                int32_t* pidx, hipStream_t st, LaunchEvents ev = {},
                                DraftSampler smp = {});
// Final RMSNorm of block rows 1..B-1 (compacted) as fp16 in the packed fragment
// layout, rows Mz..Mpad-1 zero (bf16 storage type).
hipError_t launch_norm_pack(const DraftDims& dd, const float* src, const float* ss, int ss_nch,
                            const void* gain, int Mpad, void* zp, hipStream_t st);
// pval2 non-null: per-tile runner-up scores as well (and the variant that tracks them).
hipError_t launch_lmhead_argmax(int dtype, int R, int V, int H, const void* Z, const void* W,
                                float* pval, int32_t* pidx, float* logits, hipStream_t st,
                                LaunchEvents ev = {}, DraftSampler smp = {},
                                float* pval2 = nullptr);
// bf16 storage, one 16-row group: Zp holds every row of the group (R <= 16) as packed
// fp16 fragments; partials for all R rows (row scales do not move an argmax).
hipError_t launch_lmhead_group(int R, int V, int H, const void* Zp, const void* W, float* pval,
                               int32_t* pidx, hipStream_t st, LaunchEvents ev = {});
// ids[o] for o < R from the ntiles partials; B > 0: the partials hold R_in rows of whole
// B-row blocks and output o takes row o % (B-1) + 1 of block o / (B-1).  pval2 non-null
// (runner-up partials): top2[o] = (best, runner-up).  A row whose best score is not finite
// gets id 0 and sets DFLASH_ERR_NONFINITE (8) in *err.
hipError_t launch_argmax_reduce(int R, int ntiles, const float* pval, const int32_t* pidx,
                                int32_t* ids, int32_t* err, hipStream_t st, int R_in = 0,
                                int B = 0, const float* pval2 = nullptr, float* top2 = nullptr);

// Raises kernel fn's dynamic-LDS limit to `bytes` on the current device, once per
// (kernel, device); safe to call from several threads.
hipError_t set_lds_limit(const void* fn, int bytes);
