// Internal launchers of the DFlash kernels (host side).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define DF_MAX_ASEG 8
#define DF_MAX_WSEG 64
#define DF_MAX_LAYERS 32

struct LayerPtrs {
  void* k[DF_MAX_LAYERS];
  void* v[DF_MAX_LAYERS];
};

// out[s][m][n] = sum_{k in split s} A[m, k] * W[n, k]   (fp32 partial sums)
//   A[m, k] = a[k / ka_w][m * lda + k % ka_w]      (K split into equal-width pointer segments)
//   W[n, k] = w[j][(n - n_off[j]) * ldw + k]        for n_off[j] <= n < n_off[j+1]
struct GemmArgs {
  int M, N, K;
  int S, kc;  // number of K splits and K extent of each (filled by plan_gemm)
  int kind;   // GEMM_* (filled by plan_gemm)
  int n_aseg, ka_w;
  long long lda, ldw;
  const void* a[DF_MAX_ASEG];
  int n_wseg;
  const void* w[DF_MAX_WSEG];
  int n_off[DF_MAX_WSEG + 1];
  float* out;
};

enum { GEMM_F32 = 0, GEMM_SKINNY1 = 1, GEMM_SKINNY2 = 2, GEMM_SKINNY4 = 3, GEMM_BIG = 4 };

// Choose the kernel and the split of K for a shape; returns S.
int plan_gemm(GemmArgs& g, int dtype);
hipError_t launch_gemm(const GemmArgs& g, int dtype, hipStream_t st);

// ---- elementwise / normalisation / attention / head ----------------------------
struct DraftDims {
  int H, Hq, Hkv, d, I, V, B, batch, max_ctx, mask_id;
  float theta, eps;
};

hipError_t launch_embed_norm(int dtype, const DraftDims& dd, const int32_t* last_tok,
                             const void* embed, const void* gain, int32_t* len, int32_t* base,
                             int32_t* err, float* X, void* h, hipStream_t st);
// X += sum_s P[s]; out = RMSNorm(X) * g  (rows [0, M)); if compact_B > 0 only rows with
// (row % compact_B) != 0 are written, packed; dbg (fp32, nullable) gets the normed rows.
hipError_t launch_residual_norm(int dtype, int M, int H, const float* P, int S, float* X,
                                const void* gain, float eps, void* out, int compact_B,
                                float* dbg, hipStream_t st);
// c = RMSNorm(sum_s P[s]) * g for fusion rows; dbg nullable.
hipError_t launch_fuse_norm(int dtype, int M, int H, const float* P, int S, const void* gain,
                            float eps, void* out, float* dbg, hipStream_t st);
hipError_t launch_qkv_post(int dtype, const DraftDims& dd, const float* P, int S,
                           const int32_t* len, void* q, void* kc, void* vc, int32_t* err,
                           hipStream_t st);
hipError_t launch_swiglu(int dtype, int M, int I, const float* P, int S, void* out,
                         hipStream_t st);
hipError_t launch_attention(int dtype, const DraftDims& dd, const void* q, const void* kc,
                            const void* vc, const int32_t* len, int n_split, float* opart,
                            float* ml, void* o, hipStream_t st);
int attention_splits(const DraftDims& dd);
// Rows of fuse_inject: per packed row p, seq[p] (-1 if unused) and pos[p].
hipError_t launch_rowmap(int total_rows, int batch, const int32_t* row_start,
                         const int32_t* row_count, const int32_t* len, int max_ctx,
                         int32_t* seq, int32_t* pos, int32_t* err, hipStream_t st);
hipError_t launch_inject_post(int dtype, int rows, int n_layers, int Hkv, int d, int max_ctx,
                              float theta, const float* P, int S, const int32_t* seq,
                              const int32_t* pos, void* const* kcs, void* const* vcs,
                              hipStream_t st);  // kcs/vcs: host arrays of n_layers device pointers
hipError_t launch_len_update(int batch, int total_rows, const int32_t* row_start,
                             const int32_t* row_count, int32_t* len, int max_ctx, int32_t* err,
                             hipStream_t st);
hipError_t launch_accept_trim(int batch, int B, const int32_t* drafts, const int32_t* targets,
                              int32_t* accept_len, int32_t* bonus, int32_t* len,
                              const int32_t* base, int32_t* err, hipStream_t st);
// lm_head + argmax over rows Z [R, H]; partial results then reduced into ids.
int lmhead_tiles(int dtype, int R, int V, int H);
hipError_t launch_lmhead_argmax(int dtype, int R, int V, int H, const void* Z, const void* W,
                                float* pval, int32_t* pidx, float* logits, hipStream_t st);
hipError_t launch_argmax_reduce(int R, int ntiles, const float* pval, const int32_t* pidx,
                                int32_t* ids, hipStream_t st);
