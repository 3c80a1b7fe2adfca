// The pipelined 256x256 MFMA tile shared by the batched GEMM and the batched
// lm_head: both operands are fp16 fragments in the packed layout (16 rows x 32
// k per 1 KB), streamed into LDS with 16-byte direct-to-LDS loads.
#pragma once

#include "common.h"

constexpr int MF_M = 256, MF_N = 256;  // output tile of a workgroup
constexpr int MF_WAVES = 8;            // 2 (M) x 4 (N) waves of 128 x 64
constexpr int MF_STG = 4;              // pipeline stages of one 32-wide k step (32 KB each)
constexpr int MF_FPW = 32 / MF_WAVES;  // 1 KB fragments each wave loads per stage
constexpr int MF_LDS = MF_STG * 32 * 1024;

typedef __attribute__((address_space(3))) void lds_void;
// Both operands stream with the non-temporal cache policy: measured at batch 32,
// per launch, gate|up 112 -> 110 us and the lm_head 593 -> 586 us (weights alone
// non-temporal, with the A rows cached: slower than either).
constexpr int MF_CPOL_NT = 2;

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
// (+ lane * 8 already applied) to fragment f = wave * MF_FPW + j at the first k
// step: f < 16 is A row group f of the tile, f >= 16 is B row group f - 16; the
// next k step of a fragment sits 512 elements further.  Stage s of smem holds the
// 32 fragments of one k step.  Wave (wm, wn) = (wave / 4, wave % 4) accumulates
// A groups 8wm.. x B groups 4wn..: acc[a][b] is the 16x16 block of rows
// 16 (8 wm + a) + 4 (lane / 16) + r, columns 16 (4 wn + b) + lane % 16.
__device__ __forceinline__ void mf_tile(const f16_t* const (&src)[MF_FPW], int nks, f16x8* smem,
                                        int wave, int lane, floatx4 (&acc)[8][4]) {
  auto issue = [&](int i) {  // k step i into stage i % MF_STG
    f16x8* st = smem + (i % MF_STG) * 32 * 64;
#pragma unroll
    for (int j = 0; j < MF_FPW; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(src[j] + (long long)i * 512),
                                       (lds_void*)(st + (wave * MF_FPW + j) * 64), 16, 0,
                                       MF_CPOL_NT);
  };
  const int wm = wave >> 2, wn = wave & 3;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < MF_STG - 1; ++i)
    if (i < nks) issue(i);
  for (int i = 0; i < nks; ++i) {
    // stage i's fragments have landed (the loads of the next MF_STG - 2 stages may
    // still be in flight)
    const int ahead = min(MF_STG - 2, nks - 1 - i);
    if (ahead >= 2) vm_wait<2 * MF_FPW>();
    else if (ahead == 1) vm_wait<MF_FPW>();
    else vm_wait<0>();
    barrier_pipelined();  // every wave's stage i is in LDS; every wave is done with stage i - 1
    if (i + MF_STG - 1 < nks) issue(i + MF_STG - 1);
    const f16x8* st = smem + (i % MF_STG) * 32 * 64;
    f16x8 af[8], bf[4];
#pragma unroll
    for (int a = 0; a < 8; ++a) af[a] = st[(8 * wm + a) * 64 + lane];
#pragma unroll
    for (int b = 0; b < 4; ++b) bf[b] = st[(16 + 4 * wn + b) * 64 + lane];
    __builtin_amdgcn_sched_barrier(0);  // all fragment reads before the MFMAs
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[a], bf[b], acc[a][b], 0, 0, 0);
  }
}
