// The pipelined MFMA tiles shared by the batched GEMM and the batched lm_head:
// both operands are fp16 fragments in the packed layout (16 rows x 32 k per 1 KB),
// streamed into LDS with 16-byte direct-to-LDS loads.
#pragma once

#include "common.h"

// Tile shapes: TM x TN outputs per workgroup, 8 waves in 2 (M) x 4 (N), each wave
// (TM / 2) x (TN / 4).  256 x 256 (waves of 128 x 64) is the most work per byte of
// LDS traffic; 128 x 128 (64 x 32) gives four times the tiles for small outputs,
// 128 x 256 (64 x 64) fits 65-128 rows, 128 x 384 (64 x 96) fills all 256 CUs with
// a 512-row gate|up GEMM that has 192 tiles of 256 x 256.
constexpr int MF_WAVES = 8;
constexpr int MF_STG = 4;  // pipeline stages of one 32-wide k step
template <int TM, int TN>
struct MfTile {
  static constexpr int FA = TM / 16;           // A fragments (row groups) of a k step
  static constexpr int FR = TM / 16 + TN / 16;  // fragments of a k step (1 KB each)
  static constexpr int FPW = FR / MF_WAVES;     // fragments each wave loads per k step
  static constexpr int AG = TM / 32;            // row groups of a wave
  static constexpr int BG = TN / 64;            // column groups of a wave
  static constexpr int LDS = MF_STG * FR * 1024;
  static_assert(FR % MF_WAVES == 0, "fragments per wave");
};
// the 256 x 256 tile
constexpr int MF_M = 256, MF_N = 256;
// GEMMs of at most this many rows take 128 x 128 tiles.  Measured per round: the
// batch-8 bulk workload (128 rows) 2.36 -> 2.10 ms with them (and the 128-row lm_head
// tile); at batch 32 (480 rows) 128 x 128 tiles for the projections with fewer than
// 128 tiles of 256 x 256 were slower (2.86 -> 2.92 ms with 256 workgroups, 3.16 with
// 512), the longer K loop per tile not paying for the lower work per LDS byte.
constexpr int MF_SMALL_ROWS = 128;
constexpr int MF_FPW = MfTile<256, 256>::FPW;
constexpr int MF_LDS = MfTile<256, 256>::LDS;

typedef __attribute__((address_space(3))) void lds_void;
// Cache policy of each operand's loads (2: non-temporal, 0: default).  The A rows are
// re-read by every column tile and each weight tile by the row tiles beside it on the
// same L2, so both keep the default.  Measured at batch 32 (round; lm_head per launch,
// rocprofv3 FETCH_SIZE / WRITE_SIZE): default / default 2.82 ms, lm_head 553 us moving
// 1.455 GB for 1.249 GB of weights; both non-temporal 2.86 ms, 556 us, 1.802 GB (the A
// rows fetched again); A default, weights non-temporal 2.85 ms, 575 us, 1.493 GB; A
// non-temporal, weights default 2.89 ms, 580 us, 1.596 GB.
constexpr int MF_CPOL_A = 0, MF_CPOL_B = 0;

// XCD-aware tile order.  Workgroups are dealt round-robin to the 8 XCDs
// (workgroup L runs on XCD L % 8), each with its own L2.  A launch of
// 8 * per_xcd workgroups gives XCD x the consecutive tiles
// [x * per_xcd, (x + 1) * per_xcd), so tiles adjacent in the caller's order
// (the row tiles that share one weight tile) run at the same time on the same
// L2 and the weight tile is fetched from HBM once.  Returns the tile index
// (>= the tile count for the padding workgroups).
__device__ __forceinline__ int xcd_tile(int per_xcd) {
  const int L = blockIdx.x;
  return (L & 7) * per_xcd + (L >> 3);
}
inline int xcd_per(int tiles) { return (tiles + 7) / 8; }

// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// acc += A_tile . B_tile^T over nks k steps.  src[j] is this wave's lane pointer
// (+ lane * 8 already applied) to fragment f = wave * FPW + j at the first k
// step: f < FA is A row group f of the tile, f >= FA is B row group f - FA; the
// next k step of a fragment sits 512 elements further.  Stage s of smem holds the
// FR fragments of one k step.  Wave (wm, wn) = (wave / 4, wave % 4) accumulates
// A groups AG wm.. x B groups BG wn..: acc[a][b] is the 16x16 block of rows
// 16 (AG wm + a) + 4 (lane / 16) + r, columns 16 (BG wn + b) + lane % 16.
template <int TM, int TN>
__device__ __forceinline__ void mf_tile(const f16_t* const (&src)[MfTile<TM, TN>::FPW], int nks,
                                        f16x8* smem, int wave, int lane,
                                        floatx4 (&acc)[MfTile<TM, TN>::AG][MfTile<TM, TN>::BG]) {
  using T = MfTile<TM, TN>;
  constexpr int FPW = T::FPW, FR = T::FR, FA = T::FA, AG = T::AG, BG = T::BG;
  auto issue = [&](int i) {  // k step i into stage i % MF_STG
    f16x8* st = smem + (i % MF_STG) * FR * 64;
#pragma unroll
    for (int j = 0; j < FPW; ++j) {
      const void* g = (const void*)(src[j] + (long long)i * 512);
      lds_void* l = (lds_void*)(st + (wave * FPW + j) * 64);
      if (wave * FPW + j < FA)  // wave-uniform
        __builtin_amdgcn_global_load_lds(g, l, 16, 0, MF_CPOL_A);
      else
        __builtin_amdgcn_global_load_lds(g, l, 16, 0, MF_CPOL_B);
    }
  };
  const int wm = wave >> 2, wn = wave & 3;
#pragma unroll
  for (int i = 0; i < AG; ++i)
#pragma unroll
    for (int j = 0; j < BG; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < MF_STG - 1; ++i)
    if (i < nks) issue(i);
  for (int i = 0; i < nks; ++i) {
    // stage i's fragments have landed (the loads of the next MF_STG - 2 stages may
    // still be in flight)
    const int ahead = min(MF_STG - 2, nks - 1 - i);
    static_assert(MF_STG <= 5, "wait counts below cover up to three stages ahead");
    if (ahead >= 3) vm_wait<3 * FPW>();
    else if (ahead == 2) vm_wait<2 * FPW>();
    else if (ahead == 1) vm_wait<FPW>();
    else vm_wait<0>();
    barrier_pipelined();  // every wave's stage i is in LDS; every wave is done with stage i - 1
    if (i + MF_STG - 1 < nks) issue(i + MF_STG - 1);
    const f16x8* st = smem + (i % MF_STG) * FR * 64;
    f16x8 af[AG], bf[BG];
#pragma unroll
    for (int a = 0; a < AG; ++a) af[a] = st[(AG * wm + a) * 64 + lane];
#pragma unroll
    for (int b = 0; b < BG; ++b) bf[b] = st[(FA + BG * wn + b) * 64 + lane];
    __builtin_amdgcn_sched_barrier(0);  // all fragment reads before the MFMAs
#pragma unroll
    for (int a = 0; a < AG; ++a)
#pragma unroll
      for (int b = 0; b < BG; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[a], bf[b], acc[a][b], 0, 0, 0);
  }
}
