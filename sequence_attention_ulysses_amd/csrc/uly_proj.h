// Private declarations of the QKV projection kernel (uly_proj.hip) shared
// with the host runtime.  Not part of the public ABI.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "fastdiv.h"

namespace uly {

// ---------------------------------------------------------------------------
// QKV projection on MFMA with the Q/K norm + RoPE + head-band store epilogue
// (uly_proj.hip).  x[M][K] holds the token rows of every rank, rank-major
// (m = (r*B + b)*S_l + s); w[N][K] the weight, N = (Hq + 2*Hkv) * 128
// output columns: q's heads, then k's, then v's.  A block computes
// kProjHeads heads (128 columns each) of kProjTileT tokens; K advances
// kProjTileK at a time.
// ---------------------------------------------------------------------------
#ifndef ULY_PROJ_WAVE_T
#define ULY_PROJ_WAVE_T 64
#endif
constexpr int kProjD = 128;          // head dim the projection kernel is built for
constexpr int kProjHeads = 2;        // heads per block, one per wave row
#ifndef ULY_PROJ_TILE_T
#define ULY_PROJ_TILE_T 256
#endif
constexpr int kProjTileT = ULY_PROJ_TILE_T;   // tokens per block
constexpr int kProjWaveT = ULY_PROJ_WAVE_T;                            // tokens per wave
constexpr int kProjThreads = kProjHeads * (kProjTileT / kProjWaveT) * 64;   // 8 waves (4 for 128)
#ifndef ULY_PROJ_TILE_K
#define ULY_PROJ_TILE_K 64
#endif
constexpr int kProjTileK = ULY_PROJ_TILE_K;   // K per LDS stage

struct ProjArgs {
    const uint16_t *x;
    const uint16_t *w;
    const uint16_t *wn[2];           // RMSNorm weights of q and k, [128]
    uint16_t *dst[3];                // targets q, k, v: [P][B][S][Hl][128]
    const float *cos_tab;            // [rows][64]
    const float *sin_tab;
    int64_t d_q[3], d_b[3], d_g[3];  // destination element strides (rank, batch, global token)
    FastDiv sl;                      // S_l
    FastDiv bdiv;                    // B
    FastDiv hl[3];                   // heads per rank of q, k, v
    FastDiv nhb;                     // head blocks per token tile: ceil((Hq + 2*Hkv) / kProjHeads)
    uint32_t M, K, S_l;
    uint32_t Hq, Hkv, NH;            // NH = Hq + 2*Hkv
    float eps, inv_D;
};

// deep_b: three-stage ring for the token rows (a token operand too large to
// stay in the caches), else two.
void launch_proj(const ProjArgs &a, int dtype, uint32_t blocks, bool deep_b, hipStream_t stream);

}  // namespace uly
