// C ABI of the DFlash draft step: argument validation (pure host code, so a
// bad call never reaches the GPU), workspace carving and the kernel sequence
// of each call.  See include/dflash.h for the contract.

#include <algorithm>
#include <cmath>
#include <mutex>
#include <set>
#include <string.h>
#include <utility>

#include "../../include/dflash.h"
#include "common.h"
#include "kernels.h"

hipError_t set_lds_limit(const void* fn, int bytes) {
  static std::mutex mu;
  static std::set<std::pair<const void*, int>> done;  // (kernel, device)
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if (done.count({fn, dev})) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.insert({fn, dev});
  return e;
}

namespace {

constexpr size_t ALIGN = 256;
constexpr int FI_CHUNK = 16384;  // rows of one fuse_inject pass

size_t up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

int esize(const dflash_config* c) { return c->dtype == DFLASH_F32 ? 4 : 2; }

int check_config(const dflash_config* c) {
  if (!c) return DFLASH_EINVAL;
  if (c->n_layers <= 0 || c->hidden <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 ||
      c->head_dim <= 0 || c->inter <= 0 || c->vocab < 2 || c->n_feat_layers <= 0 ||
      c->feat_hidden <= 0)
    return DFLASH_EINVAL;
  if (c->n_q_heads % c->n_kv_heads) return DFLASH_EINVAL;
  if (c->dtype != DFLASH_F32 && c->dtype != DFLASH_BF16) return DFLASH_ERANGE;
  if (c->head_dim != 64 && c->head_dim != 128) return DFLASH_ERANGE;
  if (c->block_max < 2 || c->block_max > 16) return DFLASH_ERANGE;
  if (c->mask_token_id < 0 || c->mask_token_id >= c->vocab) return DFLASH_EINVAL;
  if (c->n_layers > DF_MAX_LAYERS || 2 * c->n_layers > DF_MAX_WSEG) return DFLASH_ERANGE;
  if (c->n_feat_layers > DF_MAX_ASEG) return DFLASH_ERANGE;
  if (!(c->rms_eps >= 0.f) || !(c->rope_theta > 0.f)) return DFLASH_EINVAL;
  const int al = c->dtype == DFLASH_BF16 ? 256 : 64;
  const int qd = c->n_q_heads * c->head_dim;
  if (c->hidden % al || qd % al || c->inter % al || c->feat_hidden % al) return DFLASH_ERANGE;
  if (c->dtype == DFLASH_BF16) {
    if (c->vocab % 16) return DFLASH_ERANGE;
    const int g = c->n_q_heads / c->n_kv_heads;
    if (g * c->block_max > 128) return DFLASH_ERANGE;
  }
  return DFLASH_OK;
}

int check_weights(const dflash_config* c, const dflash_weights* w, bool need_layers_full) {
  if (!w) return DFLASH_EINVAL;
  const int want = c->dtype == DFLASH_BF16 ? DFLASH_LAYOUT_PACKED : DFLASH_LAYOUT_ROWMAJOR;
  if (w->layout != want) return DFLASH_EINVAL;
  if (!w->embed || !w->fc || !w->fc_norm || !w->final_norm || !w->lm_head) return DFLASH_EINVAL;
  const void* const* arrs[] = {w->in_norm, w->wq, w->wk, w->wv, w->wo,
                               w->post_norm, w->w_gate, w->w_up, w->w_down};
  for (int i = 0; i < 9; ++i) {
    const bool needed = need_layers_full || i == 2 || i == 3;  // injection needs wk, wv
    if (!needed) continue;
    if (!arrs[i]) return DFLASH_EINVAL;
    for (int l = 0; l < c->n_layers; ++l)
      if (!arrs[i][l]) return DFLASH_EINVAL;
  }
  return DFLASH_OK;
}

int check_kv(const dflash_config* c, const dflash_kv* kv) {
  if (!kv || !kv->k || !kv->v || !kv->len || !kv->base || !kv->err) return DFLASH_EINVAL;
  if (kv->batch <= 0) return DFLASH_EINVAL;
  if (kv->max_ctx < 64 || kv->max_ctx % 64) return DFLASH_ERANGE;
  for (int l = 0; l < c->n_layers; ++l)
    if (!kv->k[l] || !kv->v[l]) return DFLASH_EINVAL;
  return DFLASH_OK;
}

DraftDims make_dims(const dflash_config* c, int batch, int block, int max_ctx) {
  DraftDims d;
  d.H = c->hidden;
  d.Hq = c->n_q_heads;
  d.Hkv = c->n_kv_heads;
  d.d = c->head_dim;
  d.I = c->inter;
  d.V = c->vocab;
  d.B = block;
  d.batch = batch;
  d.max_ctx = max_ctx;
  d.mask_id = c->mask_token_id;
  d.theta = c->rope_theta;
  d.eps = c->rms_eps;
  return d;
}

GemmArgs gemm_shape(int M, int N, int K) {
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  g.M = M;
  g.N = N;
  g.K = K;
  return g;
}

// ---- workspace plans ------------------------------------------------------------------------
// Every projection is a GEMM storing fp32 partial sums over its K splits; the
// column-parallel row kernels that consume them reduce the splits in order and
// apply the epilogue (residual, SwiGLU, RoPE + cache write).
// Which kernels a draft of M = batch * block rows runs (they depend on the shape only):
// one 16-row group (batch-1 drafting) takes full-K GEMMs that add into X
// themselves, fed packed fp16 A rows by the attention merge and by SwiGLU.
struct DraftPath {
  bool rowk_o, rowk_d, rowk_gu, rowk_qkv;
};

DraftPath draft_path(const dflash_config* c, int M) {
  const int H = c->hidden, QD = c->n_q_heads * c->head_dim, I = c->inter;
  DraftPath p;
  const bool bf = c->dtype == DFLASH_BF16;
  p.rowk_o = bf && rowk_fits(M, H, QD, false);
  p.rowk_d = bf && rowk_fits(M, H, I, false);
  // ... and gate/up too, with SwiGLU in its epilogue: the output projection then
  // also writes gate/up's A rows, scaled per row (statistics after it go to ss2)
  // (the down projection then takes its full-K GEMM as well, so it must fit too)
  p.rowk_gu = p.rowk_o && p.rowk_d && rowk_fits(M, I, H, true) && H % 1024 == 0 && H <= 8192;
  // ... and QKV too, with RoPE and the cache write in its epilogue: the embedding
  // and the down projection then write its A rows
  p.rowk_qkv = p.rowk_gu && rowk_qkv_fits(M, H, c->head_dim);
  return p;
}

struct DraftPlan {
  size_t X, ss, ss2, sc, y, rope, q, o, a, z, P, apack, opart, pval, pidx, pval2, total;
  int ntiles;
};

// generic: the plan of the causal passes (target verification, input-fusion
// injection), which run every projection through the split GEMMs
DraftPlan plan_draft(const dflash_config* c, int batch, int block, int max_ctx,
                     bool generic = false) {
  DraftPlan p;
  const int M = batch * block, Mz = batch * (block - 1);
  const int H = c->hidden, QD = c->n_q_heads * c->head_dim, KVD = c->n_kv_heads * c->head_dim;
  const int I = c->inter;
  const int es = esize(c);
  DraftDims dd = make_dims(c, batch, block, max_ctx);
  const DraftPath path = generic ? DraftPath{false, false, false, false} : draft_path(c, M);
  size_t pmax = 0, amax = 0;
  // the projections that run as split GEMMs (partial sums in P, packed A rows in apack)
  const int shapes[4][2] = {{QD + 2 * KVD, H}, {H, QD}, {2 * I, H}, {H, I}};
  const bool full_k[4] = {path.rowk_qkv, path.rowk_o, path.rowk_gu, path.rowk_d};
  for (int i = 0; i < 4; ++i) {
    if (full_k[i]) continue;
    GemmArgs g = gemm_shape(M, shapes[i][0], shapes[i][1]);
    g.a_f32 = 1;
    g.ka_w = shapes[i][1];
    plan_gemm(g, c->dtype);
    const size_t need = (size_t)g.S * M * shapes[i][0];
    if (need > pmax) pmax = need;
    if (gemm_apack_bytes(g) > amax) amax = gemm_apack_bytes(g);
  }
  // lm_head partial tiles: the most any head variant this shape can take writes
  // (greedy, logits stored, runner-up tracked; the 16-row group head keeps every row)
  p.ntiles = lmhead_tiles(c->dtype, Mz, c->vocab, H, true);
  const int alt[4] = {lmhead_tiles(c->dtype, Mz, c->vocab, H, false),
                      lmhead_tiles(c->dtype, Mz, c->vocab, H, false, true),
                      lmhead_tiles(c->dtype, M, c->vocab, H, false),
                      lmhead_tiles(c->dtype, M, c->vocab, H, true)};  // a verification's rows
  for (int t : alt)
    if (t > p.ntiles) p.ntiles = t;
  if (c->dtype == DFLASH_BF16 && Mz > 16) {  // packed final-norm rows of the batched lm_head
    const size_t zb = (size_t)((Mz + 255) / 256 * 256) * H * 2;
    if (zb > amax) amax = zb;
  }
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += up(bytes);
    return o;
  };
  p.X = take((size_t)M * H * 4);
  p.ss = take((size_t)M * ss_chunks(H) * 4);
  // one 16-row group: the statistics after the attention sublayer, the per-row
  // scale and the packed rows the full-K output projection hands to gate/up
  const bool group = M <= 16;
  p.ss2 = take(group ? (size_t)M * ss_chunks(H) * 4 : 0);
  p.sc = take(group ? 16 * 4 : 0);
  p.y = take(group ? (size_t)16 * H * 2 : 0);
  p.rope = take((size_t)M * c->head_dim * 4);
  p.q = take((size_t)M * QD * 4);
  // attention output: fp32 rows, or fp16 packed rows padded to 256 (batched path)
  const size_t o32 = (size_t)M * QD * 4, o16 = (size_t)((M + 255) / 256 * 256) * QD * 2;
  p.o = take(o32 > o16 ? o32 : o16);
  // SwiGLU output: fp32 rows, or fp16 packed rows padded to 256 (batched path)
  const size_t a32 = (size_t)M * I * 4, a16 = (size_t)((M + 255) / 256 * 256) * I * 2;
  p.a = take(a32 > a16 ? a32 : a16);
  p.z = take((size_t)M * H * es);  // normalised rows for the lm_head (every row of a verification)
  p.P = take(pmax * 4);
  p.apack = take(amax);
  // attention partials
  p.opart = take(attention_part_bytes(c->dtype == DFLASH_F32 ? 0 : 1, dd));
  p.pval = take((size_t)p.ntiles * M * 4);  // M >= Mz: the 16-row group head keeps every row
  p.pidx = take((size_t)p.ntiles * M * 4);
  p.pval2 = take((size_t)p.ntiles * M * 4);  // runner-up partials (top-2 parity output)
  p.total = off;
  return p;
}

struct FusePlan {
  size_t seq, pos, Pf, y, ss, Pi, apack, total;
  int chunk;
};

FusePlan plan_fuse(const dflash_config* c, int total_rows) {
  FusePlan p;
  const int R = total_rows < FI_CHUNK ? total_rows : FI_CHUNK;
  p.chunk = R;
  const int H = c->hidden, KVD = c->n_kv_heads * c->head_dim;
  const int NI = c->n_layers * 2 * KVD;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += up(bytes);
    return o;
  };
  p.seq = take((size_t)total_rows * 4);
  p.pos = take((size_t)total_rows * 4);
  size_t sf = 0, si = 0, amax = 0;
  // partial sizes depend on the row count of a pass: take the max over pass sizes that occur
  const int counts[2] = {R, total_rows % FI_CHUNK};
  for (int rc : counts) {
    if (rc <= 0) continue;
    GemmArgs gf = gemm_shape(rc, H, c->n_feat_layers * c->feat_hidden);
    gf.ka_w = c->feat_hidden;
    plan_gemm(gf, c->dtype);
    GemmArgs gi = gemm_shape(rc, NI, H);
    gi.a_f32 = 1;
    gi.ka_w = H;
    plan_gemm(gi, c->dtype);
    if (gemm_apack_bytes(gf) > amax) amax = gemm_apack_bytes(gf);
    if (gemm_apack_bytes(gi) > amax) amax = gemm_apack_bytes(gi);
    if ((size_t)gf.S * rc * H > sf) sf = (size_t)gf.S * rc * H;
    if ((size_t)gi.S * rc * NI > si) si = (size_t)gi.S * rc * NI;
  }
  p.Pf = take(sf * 4);
  p.y = take((size_t)R * H * 4);
  p.ss = take((size_t)R * ss_chunks(H) * 4);
  p.Pi = take(si * 4);
  p.apack = take(amax);
  p.total = off;
  return p;
}

// Workspace that covers every fuse_inject call of up to max_rows rows: a call of
// T rows runs passes of min(T, FI_CHUNK) rows and T % FI_CHUNK rows, whose split
// partials and packed rows do not grow monotonically with the row count, so each
// buffer is sized for the largest need of any pass size <= min(max_rows, FI_CHUNK).
size_t fuse_envelope_bytes(const dflash_config* c, int max_rows) {
  const int R = max_rows < FI_CHUNK ? max_rows : FI_CHUNK;
  const int H = c->hidden, KVD = c->n_kv_heads * c->head_dim;
  const int NI = c->n_layers * 2 * KVD;
  size_t sf = 0, si = 0, amax = 0;
  for (int rc = 1; rc <= R; ++rc) {
    GemmArgs gf = gemm_shape(rc, H, c->n_feat_layers * c->feat_hidden);
    gf.ka_w = c->feat_hidden;
    plan_gemm(gf, c->dtype);
    GemmArgs gi = gemm_shape(rc, NI, H);
    gi.a_f32 = 1;
    gi.ka_w = H;
    plan_gemm(gi, c->dtype);
    if (gemm_apack_bytes(gf) > amax) amax = gemm_apack_bytes(gf);
    if (gemm_apack_bytes(gi) > amax) amax = gemm_apack_bytes(gi);
    if ((size_t)gf.S * rc * H > sf) sf = (size_t)gf.S * rc * H;
    if ((size_t)gi.S * rc * NI > si) si = (size_t)gi.S * rc * NI;
  }
  // the same buffers, in the same order, as plan_fuse
  return up((size_t)max_rows * 4) * 2 + up(sf * 4) + up((size_t)R * H * 4) +
         up((size_t)R * ss_chunks(H) * 4) + up(si * 4) + up(amax);
}

inline char* wsp(void* ws, size_t off) { return (char*)ws + off; }

// Timing hook of dflash_debug: the next event pair for a launch of class `cls`
// (recorded by the dispatch itself at kernel start and end), or none.
struct Timer {
  dflash_debug* d;
  LaunchEvents take(int cls) {
    if (!d || d->timed != cls || !d->events || 2 * d->n_used + 1 >= d->n_events) return {};
    LaunchEvents e;
    e.start = (hipEvent_t)d->events[2 * d->n_used];
    e.stop = (hipEvent_t)d->events[2 * d->n_used + 1];
    d->n_used++;
    return e;
  }
};

#define HIPCHK(x)                         \
  do {                                    \
    if ((x) != hipSuccess) return DFLASH_EHIP; \
  } while (0)

}  // namespace

extern "C" {

size_t dflash_workspace_bytes(const dflash_config* cfg, int32_t batch, int32_t max_rows,
                              int32_t max_ctx) {
  if (check_config(cfg) != DFLASH_OK || batch <= 0 || max_rows < 0 || max_ctx < 64) return 0;
  // every block a draft may take: the buffers of a smaller block can be larger
  // (another GEMM split, another attention cut)
  size_t a = 0;
  for (int blk = 1; blk <= cfg->block_max; ++blk) {  // and the causal passes' blocks
    const size_t t = std::max(blk >= 2 ? plan_draft(cfg, batch, blk, max_ctx).total : 0,
                              plan_draft(cfg, batch, blk, max_ctx, true).total);
    if (t > a) a = t;
  }
  const size_t b = fuse_envelope_bytes(cfg, max_rows);
  return a > b ? a : b;
}

int dflash_pack_weight(const void* src, int32_t n, int32_t k, void* dst, int32_t* n_overflow,
                       void* stream) {
  if (!src || !dst || n <= 0 || k <= 0) return DFLASH_EINVAL;
  if (n % 16 || k % 32) return DFLASH_ERANGE;
  HIPCHK(launch_pack_weight(src, n, k, dst, n_overflow, (hipStream_t)stream));
  return DFLASH_OK;
}

int dflash_pack_weights(const dflash_config* cfg, const dflash_weights* src,
                        const dflash_weights* dst, int32_t* n_overflow, void* stream) {
  int rc;
  if ((rc = check_config(cfg)) != DFLASH_OK) return rc;
  if (cfg->dtype != DFLASH_BF16) return DFLASH_ERANGE;
  if (!src || !dst || src->layout != DFLASH_LAYOUT_ROWMAJOR || dst->layout != DFLASH_LAYOUT_PACKED)
    return DFLASH_EINVAL;
  const int H = cfg->hidden, QD = cfg->n_q_heads * cfg->head_dim;
  const int KVD = cfg->n_kv_heads * cfg->head_dim, I = cfg->inter;
  struct Mat {
    const void* s;
    const void* d;
    int n, k;
  };
  Mat mats[2 + 7 * DF_MAX_LAYERS];
  int nm = 0;
  mats[nm++] = {src->lm_head, dst->lm_head, cfg->vocab, H};
  if (src->fc || dst->fc)  // absent in both: a target model, which has no fusion
    mats[nm++] = {src->fc, dst->fc, H, cfg->n_feat_layers * cfg->feat_hidden};
  const void* const* sl[7] = {src->wq, src->wk, src->wv, src->wo, src->w_gate, src->w_up,
                              src->w_down};
  const void* const* dl[7] = {dst->wq, dst->wk, dst->wv, dst->wo, dst->w_gate, dst->w_up,
                              dst->w_down};
  const int shp[7][2] = {{QD, H}, {KVD, H}, {KVD, H}, {H, QD}, {I, H}, {I, H}, {H, I}};
  for (int f = 0; f < 7; ++f) {
    if (!sl[f] || !dl[f]) return DFLASH_EINVAL;
    for (int l = 0; l < cfg->n_layers; ++l) mats[nm++] = {sl[f][l], dl[f][l], shp[f][0], shp[f][1]};
  }
  for (int i = 0; i < nm; ++i) {
    if (!mats[i].s || !mats[i].d || mats[i].s == mats[i].d) return DFLASH_EINVAL;
    if (mats[i].n % 16 || mats[i].k % 32) return DFLASH_ERANGE;
  }
  for (int i = 0; i < nm; ++i)
    HIPCHK(launch_pack_weight(mats[i].s, mats[i].n, mats[i].k, (void*)mats[i].d, n_overflow,
                              (hipStream_t)stream));
  return DFLASH_OK;
}

const char* dflash_strerror(int code) {
  switch (code) {
    case DFLASH_OK: return "ok";
    case DFLASH_EINVAL: return "invalid argument (null pointer or inconsistent dimensions)";
    case DFLASH_ERANGE: return "unsupported size (block, head_dim, dtype or alignment)";
    case DFLASH_ENOSPC: return "workspace too small (or, without a workspace, larger than the scratch)";
    case DFLASH_EHIP: return "HIP launch failed";
    default: return "unknown error";
  }
}

int dflash_fuse_inject(const dflash_config* cfg, const dflash_weights* w,
                       const void* const* feats, const int32_t* row_start,
                       const int32_t* row_count, int32_t total_rows, dflash_kv* kv, void* ws,
                       size_t ws_bytes, dflash_debug* dbg, void* stream) {
  int rc;
  if ((rc = check_config(cfg)) != DFLASH_OK) return rc;
  if ((rc = check_weights(cfg, w, false)) != DFLASH_OK) return rc;
  if ((rc = check_kv(cfg, kv)) != DFLASH_OK) return rc;
  if (!row_start || !row_count || total_rows < 0) return DFLASH_EINVAL;
  if (total_rows > 0) {
    if (!feats) return DFLASH_EINVAL;
    for (int i = 0; i < cfg->n_feat_layers; ++i)
      if (!feats[i]) return DFLASH_EINVAL;
  }
  const FusePlan pl = plan_fuse(cfg, total_rows);
  if (pl.total > 0 && !ws) return DFLASH_EINVAL;
  if (ws_bytes < pl.total) return DFLASH_ENOSPC;

  hipStream_t st = (hipStream_t)stream;
  Timer tm{dbg};
  const int dt = cfg->dtype, es = esize(cfg);
  const int H = cfg->hidden, KVD = cfg->n_kv_heads * cfg->head_dim;
  const int Ht = cfg->feat_hidden, NI = cfg->n_layers * 2 * KVD;
  int32_t* seq = (int32_t*)wsp(ws, pl.seq);
  int32_t* pos = (int32_t*)wsp(ws, pl.pos);
  float* Pf = (float*)wsp(ws, pl.Pf);
  float* ybuf = (float*)wsp(ws, pl.y);
  float* ssb = (float*)wsp(ws, pl.ss);
  float* Pi = (float*)wsp(ws, pl.Pi);

  if (total_rows > 0) {
    for (int r0 = 0; r0 < total_rows; r0 += FI_CHUNK) {
      const int R = total_rows - r0 < FI_CHUNK ? total_rows - r0 : FI_CHUNK;
      GemmArgs gf = gemm_shape(R, H, cfg->n_feat_layers * Ht);
      gf.n_aseg = cfg->n_feat_layers;
      gf.ka_w = Ht;
      gf.lda = Ht;
      for (int i = 0; i < cfg->n_feat_layers; ++i)
        gf.a[i] = (const char*)feats[i] + (size_t)r0 * Ht * es;
      gf.n_wseg = 1;
      gf.w[0] = w->fc;
      gf.n_off[0] = 0;
      gf.n_off[1] = H;
      gf.ldw = (long long)cfg->n_feat_layers * Ht;
      gf.out = Pf;
      plan_gemm(gf, dt);
      gf.apack = (uint16_t*)wsp(ws, pl.apack);
      HIPCHK(launch_gemm(gf, dt, st, tm.take(DFLASH_TIME_GEMM)));
      // the reduce also writes the pass's row map (read by the injection epilogue;
      // len moves only after the last pass) and, for matrix-core passes, the
      // injection GEMM's packed A rows
      const RowMap rm{kv->batch, kv->max_ctx, r0, row_start, row_count, kv->len, seq + r0,
                      pos + r0, kv->err};
      const bool y_packed = gf.kind == GEMM_MFMA;
      if (y_packed)
        HIPCHK(launch_reduce_pack(R, H, Pf, gf.S, ybuf, false, ssb, w->fc_norm, cfg->rms_eps,
                                  wsp(ws, pl.apack), st, &rm));
      else
        HIPCHK(launch_reduce_rows(R, H, Pf, gf.S, ybuf, false, ssb, st, &rm));
      if (dbg && dbg->fused)
        HIPCHK(launch_norm_rows(dt, R, H, ybuf, ssb, ss_chunks(H), w->fc_norm, cfg->rms_eps,
                                nullptr, 0, dbg->fused + (size_t)r0 * H, st));
      GemmArgs gi = gemm_shape(R, NI, H);
      gi.a_f32 = 1;
      gi.n_aseg = 1;
      gi.ka_w = H;
      gi.lda = H;
      gi.a[0] = ybuf;
      gi.nss = ssb;
      gi.nss_chunks = ss_chunks(H);
      gi.ngain = w->fc_norm;
      gi.neps = cfg->rms_eps;
      gi.n_wseg = 2 * cfg->n_layers;
      for (int l = 0; l < cfg->n_layers; ++l) {
        gi.w[2 * l] = w->wk[l];
        gi.w[2 * l + 1] = w->wv[l];
        gi.n_off[2 * l] = 2 * l * KVD;
        gi.n_off[2 * l + 1] = (2 * l + 1) * KVD;
      }
      gi.n_off[2 * cfg->n_layers] = NI;
      gi.ldw = H;
      gi.out = Pi;
      plan_gemm(gi, dt);
      gi.apack = (uint16_t*)wsp(ws, pl.apack);
      if (y_packed) {
        if (gi.kind != GEMM_MFMA) return DFLASH_EHIP;
        gi.a_packed = 1;
      }
      HIPCHK(launch_gemm(gi, dt, st, tm.take(DFLASH_TIME_GEMM)));
      const bool last = r0 + R >= total_rows;  // the last pass also advances len
      HIPCHK(launch_inject_post(dt, R, cfg->n_layers, cfg->n_kv_heads, cfg->head_dim, kv->max_ctx,
                                cfg->rope_theta, Pi, gi.S, seq + r0, pos + r0, kv->k, kv->v, st,
                                kv->batch, total_rows, row_start, row_count,
                                last ? kv->len : nullptr, kv->err));
    }
  } else {
    HIPCHK(launch_len_update(kv->batch, total_rows, row_start, row_count, kv->len, kv->max_ctx,
                             kv->err, st));
  }
  return DFLASH_OK;
}

static int draft_block(const dflash_config* cfg, const dflash_weights* w, dflash_kv* kv,
                       const int32_t* last_tok, int32_t block, const dflash_sampling* smp,
                       int32_t* draft_ids, void* ws, size_t ws_bytes, dflash_debug* dbg,
                       void* stream);

int dflash_draft_block(const dflash_config* cfg, const dflash_weights* w, dflash_kv* kv,
                       const int32_t* last_tok, int32_t block, int32_t* draft_ids, void* ws,
                       size_t ws_bytes, dflash_debug* dbg, void* stream) {
  return draft_block(cfg, w, kv, last_tok, block, nullptr, draft_ids, ws, ws_bytes, dbg, stream);
}

int dflash_draft_block_sampled(const dflash_config* cfg, const dflash_weights* w, dflash_kv* kv,
                               const int32_t* last_tok, int32_t block,
                               const dflash_sampling* smp, int32_t* draft_ids, void* ws,
                               size_t ws_bytes, dflash_debug* dbg, void* stream) {
  if (smp && !std::isfinite(smp->temperature)) return DFLASH_EINVAL;  // NaN or infinite
  if (smp && (smp->offset >> 32)) return DFLASH_EINVAL;               // a 32-bit counter word
  return draft_block(cfg, w, kv, last_tok, block, smp, draft_ids, ws, ws_bytes, dbg, stream);
}

static int draft_block(const dflash_config* cfg, const dflash_weights* w, dflash_kv* kv,
                       const int32_t* last_tok, int32_t block, const dflash_sampling* smp,
                       int32_t* draft_ids, void* ws, size_t ws_bytes, dflash_debug* dbg,
                       void* stream) {
  int rc;
  if ((rc = check_config(cfg)) != DFLASH_OK) return rc;
  if ((rc = check_weights(cfg, w, true)) != DFLASH_OK) return rc;
  if ((rc = check_kv(cfg, kv)) != DFLASH_OK) return rc;
  if (!last_tok || !draft_ids) return DFLASH_EINVAL;
  if (block < 2 || block > cfg->block_max) return DFLASH_ERANGE;
  const int batch = kv->batch;
  const DraftPlan pl = plan_draft(cfg, batch, block, kv->max_ctx);
  if (!ws) return DFLASH_EINVAL;
  if (ws_bytes < pl.total) return DFLASH_ENOSPC;

  hipStream_t st = (hipStream_t)stream;
  Timer tm{dbg};
  const int dt = cfg->dtype;
  const int M = batch * block, Mz = batch * (block - 1);
  const int H = cfg->hidden, QD = cfg->n_q_heads * cfg->head_dim;
  const int KVD = cfg->n_kv_heads * cfg->head_dim, I = cfg->inter;
  const DraftDims dd = make_dims(cfg, batch, block, kv->max_ctx);
  float* X = (float*)wsp(ws, pl.X);
  float* ss = (float*)wsp(ws, pl.ss);
  float* rope = (float*)wsp(ws, pl.rope);
  float* q = (float*)wsp(ws, pl.q);
  float* o = (float*)wsp(ws, pl.o);
  float* a = (float*)wsp(ws, pl.a);
  void* z = wsp(ws, pl.z);
  float* P = (float*)wsp(ws, pl.P);
  float* opart = (float*)wsp(ws, pl.opart);
  float* pval = (float*)wsp(ws, pl.pval);
  int32_t* pidx = (int32_t*)wsp(ws, pl.pidx);


  // batched matrix-core path: the residual reduces also write the next GEMM's
  // normalised, packed A rows (that GEMM then needs no packing pass)
  const bool batched = dt == DFLASH_BF16 && M > 64;
  bool x_packed = false;  // the next QKV GEMM's A rows are in pl.apack
  const DraftPath path = draft_path(cfg, M);
  const bool rowk_o = path.rowk_o, rowk_d = path.rowk_d, rowk_gu = path.rowk_gu;
  const bool rowk_qkv = path.rowk_qkv;
  // ... and the last one the lm_head's, scaled per row (an argmax does not see a
  // positive row scale), unless the logits themselves or the runner-up are asked
  // for, or the group's rows do not fit the head's LDS (sampling needs the true
  // logits: a row scale would change the temperature)
  DraftSampler sampler;
  // a temperature so small that its inverse overflows is the greedy limit
  if (smp && smp->temperature > 0.f && std::isfinite(1.f / smp->temperature)) {
    sampler.inv_t = 1.f / smp->temperature;
    sampler.k0 = (uint32_t)smp->seed;
    sampler.k1 = (uint32_t)(smp->seed >> 32);
    sampler.offset = (uint32_t)smp->offset;
    sampler.base = kv->base;
    sampler.rows_per_seq = block - 1;
  }
  const bool want_top2 = dbg && dbg->top2;
  const bool group_head = rowk_qkv && !(dbg && dbg->logits) && !want_top2 &&
                          sampler.inv_t == 0.f && lmhead_group_fits(M, H);
  float* ss2 = (float*)wsp(ws, pl.ss2);
  float* sc = (float*)wsp(ws, pl.sc);
  void* y = wsp(ws, pl.y);
  if (rowk_qkv)
    HIPCHK(launch_embed(dt, dd, last_tok, w->embed, kv->len, kv->base, kv->err, X, ss, rope, st,
                        w->in_norm[0], sc, y));
  else
    HIPCHK(launch_embed(dt, dd, last_tok, w->embed, kv->len, kv->base, kv->err, X, ss, rope, st));
  for (int l = 0; l < cfg->n_layers; ++l) {
    void* kl = kv->k[l];
    void* vl = kv->v[l];
    if (rowk_qkv) {  // Q | K | V of RMSNorm(X) * in_norm; RoPE and the block K/V in the cache tail
      HIPCHK(launch_rowk_qkv(y, w->wq[l], w->wk[l], w->wv[l], M, H, block, cfg->n_q_heads,
                             cfg->n_kv_heads, cfg->head_dim, ss, cfg->rms_eps, sc, kv->len, rope,
                             q, kl, vl, kv->max_ctx, st, tm.take(DFLASH_TIME_GEMM)));
    } else {  // the same through the split-K GEMM and its epilogue kernel
      GemmArgs g = gemm_shape(M, QD + 2 * KVD, H);
      g.a_f32 = 1;
      g.n_aseg = 1;
      g.ka_w = H;
      g.lda = H;
      g.a[0] = X;
      g.nss = ss;
      g.nss_chunks = ss_chunks(H);
      g.ngain = w->in_norm[l];
      g.neps = cfg->rms_eps;
      g.n_wseg = 3;
      g.w[0] = w->wq[l];
      g.w[1] = w->wk[l];
      g.w[2] = w->wv[l];
      g.n_off[0] = 0;
      g.n_off[1] = QD;
      g.n_off[2] = QD + KVD;
      g.n_off[3] = QD + 2 * KVD;
      g.ldw = H;
      g.out = P;
      plan_gemm(g, dt);
      g.apack = (uint16_t*)wsp(ws, pl.apack);
      if (x_packed) {
        if (g.kind != GEMM_MFMA) return DFLASH_EHIP;
        g.a_packed = 1;
      }
      HIPCHK(launch_gemm(g, dt, st, tm.take(DFLASH_TIME_GEMM)));
      HIPCHK(launch_qkv_post(dt, dd, P, g.S, kv->len, rope, q, kl, vl, st));
    }
    GemmArgs go = gemm_shape(M, H, QD);
    go.a_f32 = 1;
    go.n_aseg = 1;
    go.ka_w = QD;
    go.lda = QD;
    go.a[0] = o;
    go.n_wseg = 1;
    go.w[0] = w->wo[l];
    go.n_off[0] = 0;
    go.n_off[1] = H;
    go.ldw = QD;
    go.out = P;
    plan_gemm(go, dt);
    go.apack = (uint16_t*)wsp(ws, pl.apack);
    // batched path: the attention merge writes o as the projection's packed A rows
    const bool o_packed = go.kind == GEMM_MFMA || rowk_o;
    if (o_packed) {
      go.apack = (uint16_t*)o;
      go.a_packed = 1;
    }
    HIPCHK(launch_attention(dt, dd, q, kl, vl, kv->len, opart, o, st,
                            tm.take(DFLASH_TIME_ATTN), o_packed ? (uint16_t*)o : nullptr));
    if (rowk_gu) {  // X += O . Wo^T, its row statistics, gate/up's A rows
      HIPCHK(launch_rowk_resid_y(o, w->wo[l], M, H, QD, X, ss2, ss, w->post_norm[l],
                                 cfg->rms_eps, sc, y, st, tm.take(DFLASH_TIME_GEMM)));
    } else if (rowk_o) {  // X += O . Wo^T and its row statistics, in the GEMM itself
      HIPCHK(launch_rowk_resid(o, w->wo[l], M, H, QD, X, ss, st, tm.take(DFLASH_TIME_GEMM)));
    } else {
      HIPCHK(launch_gemm(go, dt, st, tm.take(DFLASH_TIME_GEMM)));
      if (batched)  // X += O . Wo^T, and the gate/up GEMM's A rows
        HIPCHK(launch_reduce_pack(M, H, P, go.S, X, true, ss, w->post_norm[l], cfg->rms_eps,
                                  wsp(ws, pl.apack), st));
      else
        HIPCHK(launch_reduce_rows(M, H, P, go.S, X, true, ss, st));  // X += O . Wo^T
    }

    if (rowk_gu) {  // SwiGLU(gate, up) as the down projection's A rows; X += MLP
      HIPCHK(launch_rowk_swiglu(y, w->w_gate[l], w->w_up[l], M, I, H, ss2, cfg->rms_eps, sc, a,
                                st, tm.take(DFLASH_TIME_GEMM)));
      const bool more = l + 1 < cfg->n_layers;
      if (rowk_qkv && (more || group_head))  // ... and the next QKV GEMM's / lm_head's A rows
        HIPCHK(launch_rowk_resid_y(a, w->w_down[l], M, H, I, X, ss, ss2,
                                   more ? w->in_norm[l + 1] : w->final_norm, cfg->rms_eps, sc, y,
                                   st, tm.take(DFLASH_TIME_GEMM)));
      else
        HIPCHK(launch_rowk_resid(a, w->w_down[l], M, H, I, X, ss, st, tm.take(DFLASH_TIME_GEMM)));
      continue;
    }
    GemmArgs gu = gemm_shape(M, 2 * I, H);
    gu.a_f32 = 1;
    gu.n_aseg = 1;
    gu.ka_w = H;
    gu.lda = H;
    gu.a[0] = X;
    gu.nss = ss;
    gu.nss_chunks = ss_chunks(H);
    gu.ngain = w->post_norm[l];
    gu.neps = cfg->rms_eps;
    gu.n_wseg = 2;
    gu.w[0] = w->w_gate[l];
    gu.w[1] = w->w_up[l];
    gu.n_off[0] = 0;
    gu.n_off[1] = I;
    gu.n_off[2] = 2 * I;
    gu.ldw = H;
    gu.out = P;
    plan_gemm(gu, dt);
    gu.apack = (uint16_t*)wsp(ws, pl.apack);
    if (batched) {
      if (gu.kind != GEMM_MFMA) return DFLASH_EHIP;
      gu.a_packed = 1;
    }
    // unsplit matrix-core GEMM: SwiGLU in its epilogue (gate and up interleaved per wave)
    // and writes it as the down projection's packed A rows
    const bool fused_swiglu = plan_swiglu(gu);
    if (fused_swiglu) gu.swiglu_out = (uint16_t*)a;
    HIPCHK(launch_gemm(gu, dt, st, tm.take(DFLASH_TIME_GEMM)));
    if (!fused_swiglu)
      HIPCHK(launch_swiglu(M, I, P, gu.S, a, st, rowk_d ? (uint16_t*)a : nullptr));
    if (rowk_d) {  // X += MLP and its row statistics
      HIPCHK(launch_rowk_resid(a, w->w_down[l], M, H, I, X, ss, st, tm.take(DFLASH_TIME_GEMM)));
      continue;
    }

    GemmArgs gd = gemm_shape(M, H, I);
    gd.a_f32 = 1;
    gd.n_aseg = 1;
    gd.ka_w = I;
    gd.lda = I;
    gd.a[0] = a;
    gd.n_wseg = 1;
    gd.w[0] = w->w_down[l];
    gd.n_off[0] = 0;
    gd.n_off[1] = H;
    gd.ldw = I;
    gd.out = P;
    plan_gemm(gd, dt);
    gd.apack = (uint16_t*)wsp(ws, pl.apack);
    if (fused_swiglu) {  // A already packed by the gate/up epilogue
      if (gd.kind != GEMM_MFMA) return DFLASH_EHIP;
      gd.apack = (uint16_t*)a;
      gd.a_packed = 1;
    }
    HIPCHK(launch_gemm(gd, dt, st, tm.take(DFLASH_TIME_GEMM)));
    if (batched) {  // X += MLP, and the next layer's QKV A rows
      const bool more = l + 1 < cfg->n_layers;
      HIPCHK(launch_reduce_pack(M, H, P, gd.S, X, true, ss, more ? w->in_norm[l + 1] : nullptr,
                                cfg->rms_eps, more ? wsp(ws, pl.apack) : nullptr, st));
      x_packed = more;
    } else {
      HIPCHK(launch_reduce_rows(M, H, P, gd.S, X, true, ss, st));  // X += MLP
    }
  }
  // final RMSNorm of rows 1..B-1 of every block, shared lm_head, argmax
  const bool want_logits = dbg && dbg->logits;
  const bool packed_head = dt == DFLASH_BF16 && Mz > 16 && !want_logits && !want_top2;
  float* pval2 = want_top2 ? (float*)wsp(ws, pl.pval2) : nullptr;
  int ntiles;
  if (group_head) {
    if (dbg && dbg->final_hidden)
      HIPCHK(launch_norm_rows(dt, M, H, X, ss, ss_chunks(H), w->final_norm, cfg->rms_eps, nullptr,
                              block, dbg->final_hidden, st));
    HIPCHK(launch_lmhead_group(M, cfg->vocab, H, y, w->lm_head, pval, pidx, st,
                               tm.take(DFLASH_TIME_LMHEAD)));
    HIPCHK(launch_argmax_reduce(Mz, lmhead_tiles(dt, M, cfg->vocab, H, false), pval, pidx,
                                draft_ids, kv->err, st, M, block));
    return DFLASH_OK;
  }
  if (packed_head) {
    if (dbg && dbg->final_hidden)
      HIPCHK(launch_norm_rows(dt, M, H, X, ss, ss_chunks(H), w->final_norm, cfg->rms_eps, nullptr,
                              block, dbg->final_hidden, st));
    void* zp = wsp(ws, pl.apack);
    HIPCHK(launch_norm_pack(dd, X, ss, ss_chunks(H), w->final_norm, (Mz + 255) / 256 * 256, zp, st));
    HIPCHK(launch_lmhead_packed(Mz, cfg->vocab, H, zp, w->lm_head, pval, pidx, st,
                                tm.take(DFLASH_TIME_LMHEAD), sampler));
    ntiles = lmhead_tiles(dt, Mz, cfg->vocab, H, false);
  } else {
    HIPCHK(launch_norm_rows(dt, M, H, X, ss, ss_chunks(H), w->final_norm, cfg->rms_eps, z, block,
                            dbg ? dbg->final_hidden : nullptr, st));
    HIPCHK(launch_lmhead_argmax(dt, Mz, cfg->vocab, H, z, w->lm_head, pval, pidx,
                                want_logits ? dbg->logits : nullptr, st, tm.take(DFLASH_TIME_LMHEAD),
                                sampler, pval2));
    ntiles = lmhead_tiles(dt, Mz, cfg->vocab, H, want_logits, want_top2);
  }
  HIPCHK(launch_argmax_reduce(Mz, ntiles, pval, pidx, draft_ids, kv->err, st, 0, 0, pval2,
                              want_top2 ? dbg->top2 : nullptr));
  return DFLASH_OK;
}

}  // extern "C"

// ---- causal passes: the synthetic target's verification, the input-fusion injection -----
namespace {

// The layers of a pass over a block of M = batch * B rows through the split GEMMs
// (or the matrix-core GEMMs at M > 64) and their epilogue kernels.  On entry the
// workspace holds X (fp32 rows), their ss partials and the RoPE table of the
// rows' positions len + dd.pos_off + r; each layer writes the block's K/V there
// (positions past max_ctx are skipped), attends causally if dd.causal, and leaves
// its output in X.  kv_only_last: the last layer stops after its K/V.  After
// layer capture[i] (ascending), X is stored in the storage type to cap_out[i].
int run_layers(const dflash_config* cfg, const dflash_weights* w, dflash_kv* kv,
               const DraftDims& dd, const DraftPlan& pl, void* ws, bool kv_only_last, int n_cap,
               const int32_t* capture, void* const* cap_out, hipStream_t st) {
  const int dt = cfg->dtype, M = dd.batch * dd.B;
  const int H = cfg->hidden, QD = cfg->n_q_heads * cfg->head_dim;
  const int KVD = cfg->n_kv_heads * cfg->head_dim, I = cfg->inter;
  float* X = (float*)wsp(ws, pl.X);
  float* ss = (float*)wsp(ws, pl.ss);
  float* rope = (float*)wsp(ws, pl.rope);
  float* q = (float*)wsp(ws, pl.q);
  float* o = (float*)wsp(ws, pl.o);
  float* a = (float*)wsp(ws, pl.a);
  float* P = (float*)wsp(ws, pl.P);
  float* opart = (float*)wsp(ws, pl.opart);
  const bool batched = dt == DFLASH_BF16 && M > 64;
  bool x_packed = false;  // the next QKV GEMM's A rows are in pl.apack
  int ci = 0;
  for (int l = 0; l < cfg->n_layers; ++l) {
    void* kl = kv->k[l];
    void* vl = kv->v[l];
    GemmArgs g = gemm_shape(M, QD + 2 * KVD, H);
    g.a_f32 = 1;
    g.n_aseg = 1;
    g.ka_w = H;
    g.lda = H;
    g.a[0] = X;
    g.nss = ss;
    g.nss_chunks = ss_chunks(H);
    g.ngain = w->in_norm[l];
    g.neps = cfg->rms_eps;
    g.n_wseg = 3;
    g.w[0] = w->wq[l];
    g.w[1] = w->wk[l];
    g.w[2] = w->wv[l];
    g.n_off[0] = 0;
    g.n_off[1] = QD;
    g.n_off[2] = QD + KVD;
    g.n_off[3] = QD + 2 * KVD;
    g.ldw = H;
    g.out = P;
    plan_gemm(g, dt);
    g.apack = (uint16_t*)wsp(ws, pl.apack);
    if (x_packed) {
      if (g.kind != GEMM_MFMA) return DFLASH_EHIP;
      g.a_packed = 1;
    }
    HIPCHK(launch_gemm(g, dt, st));
    HIPCHK(launch_qkv_post(dt, dd, P, g.S, kv->len, rope, q, kl, vl, st));
    if (kv_only_last && l + 1 == cfg->n_layers) break;

    GemmArgs go = gemm_shape(M, H, QD);
    go.a_f32 = 1;
    go.n_aseg = 1;
    go.ka_w = QD;
    go.lda = QD;
    go.a[0] = o;
    go.n_wseg = 1;
    go.w[0] = w->wo[l];
    go.n_off[0] = 0;
    go.n_off[1] = H;
    go.ldw = QD;
    go.out = P;
    plan_gemm(go, dt);
    go.apack = (uint16_t*)wsp(ws, pl.apack);
    const bool o_packed = go.kind == GEMM_MFMA;
    if (o_packed) {
      go.apack = (uint16_t*)o;
      go.a_packed = 1;
    }
    HIPCHK(launch_attention(dt, dd, q, kl, vl, kv->len, opart, o, st, {},
                            o_packed ? (uint16_t*)o : nullptr));
    HIPCHK(launch_gemm(go, dt, st));
    if (batched)
      HIPCHK(launch_reduce_pack(M, H, P, go.S, X, true, ss, w->post_norm[l], cfg->rms_eps,
                                wsp(ws, pl.apack), st));
    else
      HIPCHK(launch_reduce_rows(M, H, P, go.S, X, true, ss, st));

    GemmArgs gu = gemm_shape(M, 2 * I, H);
    gu.a_f32 = 1;
    gu.n_aseg = 1;
    gu.ka_w = H;
    gu.lda = H;
    gu.a[0] = X;
    gu.nss = ss;
    gu.nss_chunks = ss_chunks(H);
    gu.ngain = w->post_norm[l];
    gu.neps = cfg->rms_eps;
    gu.n_wseg = 2;
    gu.w[0] = w->w_gate[l];
    gu.w[1] = w->w_up[l];
    gu.n_off[0] = 0;
    gu.n_off[1] = I;
    gu.n_off[2] = 2 * I;
    gu.ldw = H;
    gu.out = P;
    plan_gemm(gu, dt);
    gu.apack = (uint16_t*)wsp(ws, pl.apack);
    if (batched) {
      if (gu.kind != GEMM_MFMA) return DFLASH_EHIP;
      gu.a_packed = 1;
    }
    const bool fused_swiglu = plan_swiglu(gu);
    if (fused_swiglu) gu.swiglu_out = (uint16_t*)a;
    HIPCHK(launch_gemm(gu, dt, st));
    if (!fused_swiglu) HIPCHK(launch_swiglu(M, I, P, gu.S, a, st));

    GemmArgs gd = gemm_shape(M, H, I);
    gd.a_f32 = 1;
    gd.n_aseg = 1;
    gd.ka_w = I;
    gd.lda = I;
    gd.a[0] = a;
    gd.n_wseg = 1;
    gd.w[0] = w->w_down[l];
    gd.n_off[0] = 0;
    gd.n_off[1] = H;
    gd.ldw = I;
    gd.out = P;
    plan_gemm(gd, dt);
    gd.apack = (uint16_t*)wsp(ws, pl.apack);
    if (fused_swiglu) {
      if (gd.kind != GEMM_MFMA) return DFLASH_EHIP;
      gd.apack = (uint16_t*)a;
      gd.a_packed = 1;
    }
    HIPCHK(launch_gemm(gd, dt, st));
    const bool more = l + 1 < cfg->n_layers;
    if (batched) {
      HIPCHK(launch_reduce_pack(M, H, P, gd.S, X, true, ss, more ? w->in_norm[l + 1] : nullptr,
                                cfg->rms_eps, more ? wsp(ws, pl.apack) : nullptr, st));
      x_packed = more;
    } else {
      HIPCHK(launch_reduce_rows(M, H, P, gd.S, X, true, ss, st));
    }
    if (ci < n_cap && capture[ci] == l) HIPCHK(launch_store_rows(dt, M, H, X, cap_out[ci++], st));
  }
  return DFLASH_OK;
}

int check_model_weights(const dflash_config* c, const dflash_weights* w) {
  if (!w) return DFLASH_EINVAL;
  const int want = c->dtype == DFLASH_BF16 ? DFLASH_LAYOUT_PACKED : DFLASH_LAYOUT_ROWMAJOR;
  if (w->layout != want || !w->embed || !w->final_norm || !w->lm_head) return DFLASH_EINVAL;
  const void* const* arrs[] = {w->in_norm, w->wq, w->wk, w->wv, w->wo,
                               w->post_norm, w->w_gate, w->w_up, w->w_down};
  for (auto arr : arrs) {
    if (!arr) return DFLASH_EINVAL;
    for (int l = 0; l < c->n_layers; ++l)
      if (!arr[l]) return DFLASH_EINVAL;
  }
  return DFLASH_OK;
}

// Buffers of an input-fusion injection of total_rows rows, in workspace order: the
// fused rows of the whole call (fp32) and their ss partials, the fusion GEMM's
// partials and packed rows for one pass (their envelope over every pass size up to
// min(total_rows, FI_CHUNK) when `envelope`), then the causal pass's own plan.
struct InputPlan {
  size_t y, yss, Pf, apack, pass, total;
  DraftPlan dp;
};

InputPlan plan_input(const dflash_config* c, int batch, int total_rows, int max_ctx, bool envelope) {
  InputPlan p;
  const int H = c->hidden;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += up(bytes);
    return o;
  };
  p.y = take((size_t)total_rows * H * 4);
  p.yss = take((size_t)total_rows * ss_chunks(H) * 4);
  const int R = total_rows < FI_CHUNK ? total_rows : FI_CHUNK;
  size_t sf = 0, amax = 0;
  auto need = [&](int rc) {
    if (rc <= 0) return;
    GemmArgs gf = gemm_shape(rc, H, c->n_feat_layers * c->feat_hidden);
    gf.ka_w = c->feat_hidden;
    plan_gemm(gf, c->dtype);
    if (gemm_apack_bytes(gf) > amax) amax = gemm_apack_bytes(gf);
    if ((size_t)gf.S * rc * H > sf) sf = (size_t)gf.S * rc * H;
  };
  if (envelope) {
    for (int rc = 1; rc <= R; ++rc) need(rc);
  } else {
    need(R);
    need(total_rows % FI_CHUNK);
  }
  p.Pf = take(sf * 4);
  p.apack = take(amax);
  p.dp = plan_draft(c, batch, c->block_max, max_ctx, true);
  p.pass = take(p.dp.total);
  p.total = off;
  return p;
}

}  // namespace

extern "C" {

int dflash_target_verify(const dflash_config* cfg, const dflash_weights* w, dflash_kv* kv,
                         const int32_t* block_ids, int32_t block, const int32_t* capture,
                         void* const* feats_out, int32_t* target_ids, void* ws, size_t ws_bytes,
                         void* stream) {
  int rc;
  if ((rc = check_config(cfg)) != DFLASH_OK) return rc;
  if ((rc = check_model_weights(cfg, w)) != DFLASH_OK) return rc;
  if ((rc = check_kv(cfg, kv)) != DFLASH_OK) return rc;
  if (!block_ids || !target_ids) return DFLASH_EINVAL;
  if (block < 1 || block > cfg->block_max) return DFLASH_ERANGE;
  const int n_cap = capture ? cfg->n_feat_layers : 0;
  for (int i = 0; i < n_cap; ++i) {
    if (capture[i] < 0 || capture[i] >= cfg->n_layers || (i && capture[i] <= capture[i - 1]))
      return DFLASH_EINVAL;
    if (!feats_out || !feats_out[i]) return DFLASH_EINVAL;
  }
  const int batch = kv->batch, M = batch * block, H = cfg->hidden;
  const DraftPlan pl = plan_draft(cfg, batch, block, kv->max_ctx, true);
  if (!ws) return DFLASH_EINVAL;
  if (ws_bytes < pl.total) return DFLASH_ENOSPC;
  hipStream_t st = (hipStream_t)stream;
  const int dt = cfg->dtype;
  DraftDims dd = make_dims(cfg, batch, block, kv->max_ctx);
  dd.causal = 1;
  float* X = (float*)wsp(ws, pl.X);
  float* ss = (float*)wsp(ws, pl.ss);
  // the block's tokens at positions len .. len + block - 1; base = len
  HIPCHK(launch_embed(dt, dd, nullptr, w->embed, kv->len, kv->base, kv->err, X, ss,
                      (float*)wsp(ws, pl.rope), st, nullptr, nullptr, nullptr, block_ids));
  if ((rc = run_layers(cfg, w, kv, dd, pl, ws, false, n_cap, capture, feats_out, st)) != DFLASH_OK)
    return rc;
  // final norm of every row, lm_head, the greedy next token of each row
  void* z = wsp(ws, pl.z);
  float* pval = (float*)wsp(ws, pl.pval);
  int32_t* pidx = (int32_t*)wsp(ws, pl.pidx);
  HIPCHK(launch_norm_rows(dt, M, H, X, ss, ss_chunks(H), w->final_norm, cfg->rms_eps, z, 0,
                          nullptr, st));
  HIPCHK(launch_lmhead_argmax(dt, M, cfg->vocab, H, z, w->lm_head, pval, pidx, nullptr, st));
  HIPCHK(launch_argmax_reduce(M, lmhead_tiles(dt, M, cfg->vocab, H, true), pval, pidx, target_ids,
                              kv->err, st));
  HIPCHK(launch_len_add(batch, block, kv->len, kv->max_ctx, kv->err, st));
  return DFLASH_OK;
}

size_t dflash_fuse_inject_input_workspace_bytes(const dflash_config* cfg, int32_t batch,
                                                int32_t max_rows, int32_t max_ctx) {
  if (check_config(cfg) != DFLASH_OK || batch <= 0 || max_rows < 0 || max_ctx < 64) return 0;
  return plan_input(cfg, batch, max_rows, max_ctx, true).total;
}

int dflash_fuse_inject_input(const dflash_config* cfg, const dflash_weights* w,
                             const void* const* feats, const int32_t* row_start,
                             const int32_t* row_count, int32_t rows_max, int32_t total_rows,
                             dflash_kv* kv, void* ws, size_t ws_bytes, dflash_debug* dbg,
                             void* stream) {
  int rc;
  if ((rc = check_config(cfg)) != DFLASH_OK) return rc;
  if ((rc = check_weights(cfg, w, true)) != DFLASH_OK) return rc;
  if ((rc = check_kv(cfg, kv)) != DFLASH_OK) return rc;
  if (!row_start || !row_count || total_rows < 0 || rows_max < 0) return DFLASH_EINVAL;
  if (total_rows > 0) {
    if (!feats) return DFLASH_EINVAL;
    for (int i = 0; i < cfg->n_feat_layers; ++i)
      if (!feats[i]) return DFLASH_EINVAL;
  }
  const int batch = kv->batch, H = cfg->hidden, B = cfg->block_max;
  const InputPlan pl = plan_input(cfg, batch, total_rows, kv->max_ctx, false);
  if (!ws) return DFLASH_EINVAL;
  if (ws_bytes < pl.total) return DFLASH_ENOSPC;
  hipStream_t st = (hipStream_t)stream;
  const int dt = cfg->dtype, es = esize(cfg), Ht = cfg->feat_hidden;
  float* y = (float*)wsp(ws, pl.y);
  float* yss = (float*)wsp(ws, pl.yss);
  // the fused rows of the whole call (the causal passes read any of them)
  for (int r0 = 0; r0 < total_rows; r0 += FI_CHUNK) {
    const int R = total_rows - r0 < FI_CHUNK ? total_rows - r0 : FI_CHUNK;
    GemmArgs gf = gemm_shape(R, H, cfg->n_feat_layers * Ht);
    gf.n_aseg = cfg->n_feat_layers;
    gf.ka_w = Ht;
    gf.lda = Ht;
    for (int i = 0; i < cfg->n_feat_layers; ++i)
      gf.a[i] = (const char*)feats[i] + (size_t)r0 * Ht * es;
    gf.n_wseg = 1;
    gf.w[0] = w->fc;
    gf.n_off[0] = 0;
    gf.n_off[1] = H;
    gf.ldw = (long long)cfg->n_feat_layers * Ht;
    gf.out = (float*)wsp(ws, pl.Pf);
    plan_gemm(gf, dt);
    gf.apack = (uint16_t*)wsp(ws, pl.apack);
    HIPCHK(launch_gemm(gf, dt, st));
    HIPCHK(launch_reduce_rows(R, H, gf.out, gf.S, y + (size_t)r0 * H, false,
                              yss + (size_t)r0 * ss_chunks(H), st));
    if (dbg && dbg->fused)
      HIPCHK(launch_norm_rows(dt, R, H, y + (size_t)r0 * H, yss + (size_t)r0 * ss_chunks(H),
                              ss_chunks(H), w->fc_norm, cfg->rms_eps, nullptr, 0,
                              dbg->fused + (size_t)r0 * H, st));
  }
  // causal passes over block_max rows of every sequence at a time
  void* pws = wsp(ws, pl.pass);
  DraftDims dd = make_dims(cfg, batch, B, kv->max_ctx);
  dd.causal = 1;
  for (int off = 0; off < rows_max && total_rows > 0; off += B) {
    dd.pos_off = off;
    HIPCHK(launch_gather_rows(dt, dd, y, yss, w->fc_norm, row_start, row_count, kv->len,
                              (float*)wsp(pws, pl.dp.X), (float*)wsp(pws, pl.dp.ss),
                              (float*)wsp(pws, pl.dp.rope), st));
    if ((rc = run_layers(cfg, w, kv, dd, pl.dp, pws, true, 0, nullptr, nullptr, st)) != DFLASH_OK)
      return rc;
  }
  HIPCHK(launch_len_update(batch, total_rows, row_start, row_count, kv->len, kv->max_ctx, kv->err,
                           st));
  return DFLASH_OK;
}

}  // extern "C"

// ---- the draft without a caller workspace ---------------------------------------------
// The workspace of dflash_draft_block_noalloc: a static device variable, so every
// GPU the library is loaded on holds its own copy for the life of the process.
// Host code never uses this name as an address (on the host it is only a
// stand-in); the device address of the current GPU's copy comes from
// hipGetSymbolAddress, once per device, and is kept in scratch_addr.
static __device__ __align__(256) unsigned char scratch[DFLASH_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int SCRATCH_DEVICES = 64;
std::once_flag scratch_once[SCRATCH_DEVICES];
void* scratch_addr[SCRATCH_DEVICES];
hipError_t scratch_status[SCRATCH_DEVICES];

// The current device's copy of `scratch`, resolved on the first call on that device.
hipError_t device_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= SCRATCH_DEVICES) return hipErrorInvalidDevice;
  std::call_once(scratch_once[dev], [dev] {
    void* p = nullptr;
    scratch_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    scratch_addr[dev] = scratch_status[dev] == hipSuccess ? p : nullptr;
  });
  *out = scratch_addr[dev];
  return scratch_status[dev];
}
}  // namespace

extern "C" {

int dflash_draft_block_noalloc(const dflash_config* cfg, const dflash_weights* w, dflash_kv* kv,
                               const int32_t* last_tok, int32_t block, int32_t* draft_ids,
                               dflash_debug* dbg, void* stream) {
  int rc;
  // the host checks of the draft come first, so a bad call touches no device state
  if ((rc = check_config(cfg)) != DFLASH_OK) return rc;
  if ((rc = check_weights(cfg, w, true)) != DFLASH_OK) return rc;
  if ((rc = check_kv(cfg, kv)) != DFLASH_OK) return rc;
  if (!last_tok || !draft_ids) return DFLASH_EINVAL;
  if (block < 2 || block > cfg->block_max) return DFLASH_ERANGE;
  if (plan_draft(cfg, kv->batch, block, kv->max_ctx).total > DFLASH_NOALLOC_SCRATCH_BYTES)
    return DFLASH_ENOSPC;
  void* ws = nullptr;
  if (device_scratch(&ws) != hipSuccess || !ws) return DFLASH_EHIP;
  return draft_block(cfg, w, kv, last_tok, block, nullptr, draft_ids, ws,
                     DFLASH_NOALLOC_SCRATCH_BYTES, dbg, stream);
}

int dflash_accept_trim(const dflash_config* cfg, const int32_t* draft_ids,
                       const int32_t* target_ids, int32_t block, int32_t* accept_len,
                       int32_t* bonus, dflash_kv* kv, void* stream) {
  int rc;
  if ((rc = check_config(cfg)) != DFLASH_OK) return rc;
  if (!kv || !kv->len || !kv->base || !kv->err || kv->batch <= 0) return DFLASH_EINVAL;
  if (!draft_ids || !target_ids || !accept_len || !bonus) return DFLASH_EINVAL;
  if (block < 2 || block > cfg->block_max) return DFLASH_ERANGE;
  HIPCHK(launch_accept_trim(kv->batch, block, draft_ids, target_ids, accept_len, bonus, kv->len,
                            kv->base, kv->err, (hipStream_t)stream));
  return DFLASH_OK;
}

}  // extern "C"
