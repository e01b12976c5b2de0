// gfx950 QKV projection with the Q/K RMSNorm + interleaved RoPE + head-band
// store in its epilogue (flashinfer PR #6332, "Description": the projection,
// the per-head norm of Q and K, the rotation and the exchange in one call;
// "Assumptions": projection, then QK-norm, then RoPE, fp32 math, 16-bit
// output).
//
// The projection is the one dense contraction of the front end, so it runs
// on the matrix cores: v_mfma_f32_16x16x32_{bf16,f16}, fp32 accumulation
// (under this chip's power limit these reach ~15 % more products per second
// on random data than v_mfma_f32_32x32x16, which also builds:
// ULY_PROJ_MFMA=32).  The product is computed transposed,
// C^T[n][t] = sum_k W[n][k] X[t][k]: both operands are K-contiguous rows,
// and the MFMA result gives each lane one token and a run of 4 head-dim
// values per 16x16 block.  The rotation pairs (2j, 2j+1) sit in one lane's
// registers; the RMSNorm of a (token, head) row is a sum over the lane's
// registers and over the token's four lane rows; exchanges across rows turn
// the runs of 4 into 16-byte stores, 64 bytes per token per instruction.
//
// Tiling: a block of 8 waves owns two heads (256 output columns; each head
// is one component q, k or v) and 256 tokens.  Wave (wn, wt) owns head wn
// and tokens [64wt, 64wt+64): a 128 x 64 tile of 8 x 4 MFMA blocks, 128
// fp32 accumulators per lane, two waves per SIMD.  (4 waves of 128 x 128,
// one per SIMD, read 2/3 of the LDS bytes per product but measured ~2 %
// slower with these products; ULY_PROJ_WAVE_T=128 builds them.)
//
// Operands go global -> LDS with global_load_lds_dwordx4 (no staging
// registers, no ds_write) into rings of 64-wide K stages, two deep for the
// weight rows and two or three deep for the token rows (three when they
// stream from HBM); later stages' loads are in flight while a stage is
// multiplied.  LDS rows are
// XOR-swizzled so the 16-byte fragment reads do not collide on banks.  The
// main loop's instruction order is fixed by hand (scheduling barriers): each
// product is followed by at most one fragment read of the next K step and
// one load of the next stage, and a stage's last K step is multiplied after
// the next barrier, while the next stage's first fragments are read.
//
// Epilogue: the block's 256 cos/sin table rows are first staged into LDS in
// one coalesced pass (as interleaved (cos, sin) pairs, rows padded by 16
// bytes), so each rotation group reads its two (cos, sin) pairs with one
// conflict-free 16-byte LDS read instead of dependent global loads.

#include <hip/hip_runtime.h>

#include "uly.h"
#include "uly_proj.h"

namespace uly {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) u32x4_t global_u32x4_t;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kWaves = kProjThreads / 64;
constexpr int kChunks = kProjTileK / 8;                  // 16-byte chunks per LDS row
constexpr int kRowsA = kProjHeads * kProjD;              // weight rows per block
constexpr int kRowsB = kProjTileT;                       // token rows per block
constexpr int kWaveT = kProjWaveT;                       // tokens per wave
#ifndef ULY_PROJ_MFMA
#define ULY_PROJ_MFMA 16
#endif
constexpr int kMf = ULY_PROJ_MFMA;                       // MFMA block edge: 16 (16x16x32) or 32 (32x32x16)
static_assert(kMf == 16 || kMf == 32, "MFMA shape");
constexpr int kKStep = 512 / kMf;                        // K per product
constexpr int kNB = kProjD / kMf;                        // head-dim blocks per wave
constexpr int kTB = kWaveT / kMf;                        // token blocks per wave
typedef float accv_t __attribute__((ext_vector_type(kMf * kMf / 64)));   // one block's accumulators per lane
constexpr int kWavesT = kProjTileT / kWaveT;             // waves along the tokens
#ifndef ULY_PROJ_WPE
#define ULY_PROJ_WPE (kWaves / 4)
#endif
constexpr int kWavesPerSimd = ULY_PROJ_WPE;              // occupancy: one block per CU by default
static_assert(kChunks == 4 || kChunks == 8, "LDS rows of 64 or 128 bytes");
static_assert(kWaves == kProjHeads * kWavesT && (kWaveT == 64 || kWaveT == 128), "wave grid");

// LDS rings: the weight rows (A) and the token rows (B) of a K stage each
// have their own ring, the stage in use plus depth-1 stages ahead.  A is
// two deep; B is two deep when the token operand stays in the caches and
// three deep (the kernel's BD parameter) when it streams from HBM: the
// weights are shared by every token tile and stay cached.
constexpr int kDepthA = 2;
constexpr int kSlotsA = kRowsA * kChunks, kSlotsB = kRowsB * kChunks;   // 16-byte slots per stage
constexpr int kInstA = kSlotsA / 64 / kWaves, kInstB = kSlotsB / 64 / kWaves;   // loads per wave per stage
static_assert(kSlotsA % (64 * kWaves) == 0 && kSlotsB % (64 * kWaves) == 0, "whole wave instructions");

// The epilogue's table: per token, 64 (cos, sin) pairs = 32 chunks, plus one
// chunk of padding so that 16 lanes reading the same chunk of 16 different
// rows start 4 banks apart and cover the 64 banks once.
constexpr int kTblRow = kProjD / 4 + 1;                  // 16-byte chunks per token row
constexpr int ring_slots(int depth_b) { return kDepthA * kSlotsA + depth_b * kSlotsB; }
constexpr int kTblSlots = kProjTileT * kTblRow;
constexpr int lds_slots(int depth_b) { return ring_slots(depth_b) > kTblSlots ? ring_slots(depth_b) : kTblSlots; }
static_assert(lds_slots(3) * 16 <= 160 * 1024, "LDS of one workgroup");

#ifndef ULY_PROJ_NT_STORE
#define ULY_PROJ_NT_STORE 0
#endif
// Output stores.  A store instruction writes 32-byte pieces of 32 rows, so
// the pieces of one line arrive from several instructions: ordinary stores
// let the L2 merge them into whole lines before they go out.
__device__ __forceinline__ void stg16(uint16_t *p, uint4 v) {
    const u32x4_t w = {v.x, v.y, v.z, v.w};
    if (ULY_PROJ_NT_STORE) __builtin_nontemporal_store(w, (global_u32x4_t *)p);
    else *(global_u32x4_t *)p = w;
}

__device__ __forceinline__ float4 ldg_f4(const float *p) {
    const u32x4_t v = *(const global_u32x4_t *)p;
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}

// Workgroup barrier for LDS hand-offs only: this thread's LDS accesses are
// complete, then s_barrier.  Unlike __syncthreads() it does not wait for
// outstanding global loads, so later stages' operand loads stay in flight
// across it.  The memory clobber keeps the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// One 16-byte-per-lane global -> LDS load into the 64 slots starting at LDS
// byte address `lds` (wave-uniform).  Issued as inline assembly so that the
// compiler's wait insertion, which would otherwise make every later LDS read
// wait for all such loads (including the stages still meant to be in
// flight), leaves it alone: the kernel orders these loads itself with
// wait_vmcnt before its barriers, and issues no other vector memory
// instruction while any is outstanding.
__device__ __forceinline__ void dma16(const void *g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(g) : "memory", "m0");
}

template <int VM>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(VM) : "memory");
}

#ifndef ULY_PROJ_GROUP
#define ULY_PROJ_GROUP 4
#endif
#ifndef ULY_PROJ_LOAD_KS
#define ULY_PROJ_LOAD_KS 1
#endif

// Block -> (token tile, head block).  Workgroups go to the 8 XCDs round
// robin (block b to XCD b % 8) and each XCD has its own L2.  The grid is cut
// into 8 contiguous runs of logical blocks, one per XCD, and logical blocks
// are ordered in groups of kGroupH head blocks x all token tiles (head
// blocks fastest), so the ~32 blocks an XCD runs at once cover about 32 /
// kGroupH token tiles and kGroupH head blocks: their X tiles and W slices
// are shared in that XCD's L2 instead of streaming per block.  A bijection
// for any grid size.
constexpr uint32_t kGroupH = ULY_PROJ_GROUP;
__device__ __forceinline__ void proj_block(const ProjArgs &a, uint32_t bid, uint32_t grid, uint32_t &tile,
                                           uint32_t &hb) {
    constexpr uint32_t kXcds = 8;
    const uint32_t q = grid / kXcds, r = grid % kXcds;
    const uint32_t x = bid % kXcds, k = bid / kXcds;
    const uint32_t L = x * q + min(x, r) + k;
    const uint32_t nhb = a.nhb.d, T = grid / nhb;
    const uint32_t g = L / (kGroupH * T), rem = L % (kGroupH * T);
    const uint32_t gh = min(kGroupH, nhb - g * kGroupH);
    tile = rem / gh;
    hb = g * kGroupH + rem % gh;
}

// LDS slot of 16-byte chunk c of row `row`.  The LDS serves a 16-byte read
// of 16 lanes in one pass over 64 four-byte banks (256 bytes): 16
// consecutive rows of 64 bytes span four bank sweeps of four rows each, so
// rows r, r+4, r+8, r+12 must use four different chunk positions; rows of
// 128 bytes sit two to a sweep, so eight rows share a set of positions.
#ifndef ULY_PROJ_SWZ
#define ULY_PROJ_SWZ (kChunks == 4 ? 2 : 1)
#endif
__device__ __forceinline__ int swz_key(int row) { return (row >> (ULY_PROJ_SWZ)) & (kChunks - 1); }
__device__ __forceinline__ int swz(int row, int c) { return row * kChunks + (c ^ swz_key(row)); }

template <int DT>
__device__ __forceinline__ accv_t mfma(uint4 a, uint4 b, accv_t c) {
#if ULY_PROJ_MFMA == 32
    if constexpr (DT == 2)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
#else
    if constexpr (DT == 2)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
#endif
}

template <int DT>
__device__ __forceinline__ float widen1(uint32_t h) {
    if constexpr (DT == 2) return __uint_as_float(h << 16);
    else return float(__builtin_bit_cast(_Float16, uint16_t(h)));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {   // one round to nearest even
    if constexpr (DT == 2) {
        bf16x2_t p = {__bf16(a), __bf16(b)};
        return __builtin_bit_cast(uint32_t, p);
    } else {
        f16x2_t p = {_Float16(a), _Float16(b)};
        return __builtin_bit_cast(uint32_t, p);
    }
}

// Global position of token row m (rank-major m = (r*B + b)*S_l + s) and its batch.
__device__ __forceinline__ uint32_t token_pos(const ProjArgs &a, uint32_t m, uint32_t &b) {
    uint32_t rb, s, r;
    a.sl.divmod(m, rb, s);
    a.bdiv.divmod(rb, r, b);
    return r * a.S_l + s;
}

// All threads of the block: the cos/sin rows of tokens m0 .. m0+255 (rows
// past M repeat token M-1) into tbl[t][...], chunk j/2 of row t holding
// (cos_j, sin_j, cos_j+1, sin_j+1) for even j.
__device__ __forceinline__ void stage_table(const ProjArgs &a, uint32_t m0, float4 *tbl, int tid) {
    constexpr int kPerRow = kProjD / 8;                  // float4 chunks of a cos (or sin) row
    constexpr int kIter = kProjTileT * kPerRow / kProjThreads;
#ifndef ULY_PROJ_TBL_BATCH
#define ULY_PROJ_TBL_BATCH 8
#endif
    constexpr int kBatch = ULY_PROJ_TBL_BATCH;
    static_assert(kIter % kBatch == 0, "batches");
#pragma unroll
    for (int u0 = 0; u0 < kIter; u0 += kBatch) {
        float4 c4[kBatch], s4[kBatch];
        int row[kBatch], q[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int idx = tid + (u0 + u) * kProjThreads;
            row[u] = idx / kPerRow;
            q[u] = idx % kPerRow;
            uint32_t b;
            const uint32_t g = token_pos(a, min(m0 + uint32_t(row[u]), a.M - 1), b);
            c4[u] = ldg_f4(a.cos_tab + size_t(g) * (kProjD / 2) + q[u] * 4);
            s4[u] = ldg_f4(a.sin_tab + size_t(g) * (kProjD / 2) + q[u] * 4);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            tbl[row[u] * kTblRow + 2 * q[u]] = make_float4(c4[u].x, s4[u].x, c4[u].y, s4[u].y);
            tbl[row[u] * kTblRow + 2 * q[u] + 1] = make_float4(c4[u].z, s4[u].z, c4[u].w, s4[u].w);
        }
    }
}

// The sum of x over lane l and lane l ^ 32: v_permlane32_swap of x with
// itself yields, in its two results, x of the lane 32 below (upper half) and
// of the lane 32 above (lower half), each beside the lane's own x.
__device__ __forceinline__ float sum_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The epilogue of wave (wn, wt) for 32 x 32 blocks (ULY_PROJ_MFMA=32):
// RMSNorm + RoPE of q/k rows (QK), or v as is, one rounding, and the stores
// into the head-sharded targets.  The head (and so QK) is wave-uniform: each
// wave runs one straight-line body.  acc[nb][tb][i] is column
// n = 32nb + 8(i/4) + 4*half + i%4 (the head-dim index d) of token
// m0 + kWaveT*wt + 32tb + lane%32 and head `hd`.
template <int DT, bool QK>
__device__ __forceinline__ void proj_epilogue(const ProjArgs &a, accv_t (&acc)[kNB][kTB], uint32_t m0,
                                              uint32_t hd, int wt, int lane, const float4 *tbl) {
    const uint32_t half = lane >> 5;
    const int comp = hd < a.Hq ? 0 : (hd < a.Hq + a.Hkv ? 1 : 2);
    const uint32_t hc = hd - (comp == 0 ? 0u : (comp == 1 ? a.Hq : a.Hq + a.Hkv));
    uint32_t qd, jd;
    a.hl[comp].divmod(hc, qd, jd);
    uint16_t *dbase = a.dst[comp] + int64_t(qd) * a.d_q[comp] + int64_t(jd) * kProjD;
    const int64_t d_b = a.d_b[comp], d_g = a.d_g[comp];

    // this lane's 64 norm weights, d = 32nb + 8grp + 4half + 0..3, widened once
    float wf[4][4][4];
    if constexpr (QK) {
        const uint16_t *wn = a.wn[comp];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                const uint2 w4 = *(const uint2 *)(wn + nb * 32 + grp * 8 + half * 4);
                wf[nb][grp][0] = widen1<DT>(w4.x & 0xFFFFu);
                wf[nb][grp][1] = widen1<DT>(w4.x >> 16);
                wf[nb][grp][2] = widen1<DT>(w4.y & 0xFFFFu);
                wf[nb][grp][3] = widen1<DT>(w4.y >> 16);
            }
    }

#pragma unroll
    for (int tb = 0; tb < kTB; ++tb) {
        const int tl = wt * kWaveT + tb * 32 + (lane & 31);   // token within the block tile
        const uint32_t tok = m0 + tl;
        const bool live = tok < a.M;
        uint32_t b;
        const uint32_t g = token_pos(a, live ? tok : a.M - 1, b);
        float inv = 1.f;
        if constexpr (QK) {
            float ss = 0.f;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int i = 0; i < 16; ++i) ss = fmaf(acc[nb][tb][i], acc[nb][tb][i], ss);
            // eps > 0 keeps the argument normal: the bare reciprocal square root suffices
            inv = __builtin_amdgcn_rsqf(fmaf(sum_halves(ss), a.inv_D, a.eps));
        }
        uint16_t *drow = dbase + int64_t(b) * d_b + int64_t(g) * d_g;
        const float4 *trow = tbl + tl * kTblRow;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            uint32_t pk[8];   // pk[2*grp + p]: the pair (d0 + 2p, d0 + 2p + 1) of register group grp
            if constexpr (QK) {
                // pairs j0 = 16nb + 4grp + 2half and j0 + 1: chunk j0 / 2 of the row;
                // the rotation in explicit fused multiply-adds, as in the exchange kernels
                float4 cs[4];
#pragma unroll
                for (int grp = 0; grp < 4; ++grp) cs[grp] = trow[nb * 8 + grp * 2 + half];
#pragma unroll
                for (int grp = 0; grp < 4; ++grp) {
                    const float cv[2] = {cs[grp].x, cs[grp].z}, sv[2] = {cs[grp].y, cs[grp].w};
#pragma unroll
                    for (int p = 0; p < 2; ++p) {
                        const int i0 = grp * 4 + p * 2;
                        const float n0 = acc[nb][tb][i0] * inv * wf[nb][grp][2 * p];
                        const float n1 = acc[nb][tb][i0 + 1] * inv * wf[nb][grp][2 * p + 1];
                        pk[grp * 2 + p] = pack2<DT>(fmaf(n0, cv[p], -(n1 * sv[p])), fmaf(n0, sv[p], n1 * cv[p]));
                    }
                }
            } else {
#pragma unroll
                for (int grp = 0; grp < 4; ++grp)
#pragma unroll
                    for (int p = 0; p < 2; ++p)
                        pk[grp * 2 + p] = pack2<DT>(acc[nb][tb][grp * 4 + p * 2], acc[nb][tb][grp * 4 + p * 2 + 1]);
            }
            // Lane half 0 holds d runs {0-3, 8-11, 16-19, 24-27} (+32nb), half 1 the
            // runs 4 higher.  v_permlane32_swap trades the upper half-wave of its
            // first operand for the lower half-wave of its second: swapping run
            // 0-3 with run 8-11 (and 16-19 with 24-27) leaves half 0 with d 0-7
            // and 16-23 and half 1 with d 8-15 and 24-31, in the same registers,
            // each a 16-byte run.
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const auto r0 = __builtin_amdgcn_permlane32_swap(pk[i], pk[2 + i], false, false);
                pk[i] = r0[0];
                pk[2 + i] = r0[1];
                const auto r1 = __builtin_amdgcn_permlane32_swap(pk[4 + i], pk[6 + i], false, false);
                pk[4 + i] = r1[0];
                pk[6 + i] = r1[1];
            }
            const uint4 lo = make_uint4(pk[0], pk[1], pk[2], pk[3]);
            const uint4 hi = make_uint4(pk[4], pk[5], pk[6], pk[7]);
            if (live) {
                stg16(drow + nb * 32 + half * 8, lo);
                stg16(drow + nb * 32 + 16 + half * 8, hi);
            }
        }
    }
}

// The sum of x over the four rows of 16 lanes that hold lane l % 16's
// token: v_permlane16_swap of x with itself pairs rows 0-1 and 2-3 (each
// lane gets its own row's x beside the partner row's), then the halves.
// Every lane of the token adds in the same order.
__device__ __forceinline__ float sum_rows4(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return sum_halves(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

// The epilogue for 16 x 16 blocks, as proj_epilogue: acc[nb][tb][r] is
// head-dim index d = 16nb + 4q + r (q = lane / 16, the lane's row) of token
// m0 + kWaveT*wt + 16tb + lane%16.  A lane holds both rotation pairs of its
// run of 4; the row's sum of squares is reduced over the token's four lane
// rows.  For the stores, the runs of two head-dim blocks are traded across
// rows (v_permlane32_swap, then v_permlane16_swap) so that row q writes 16
// bytes of one of them: each store instruction covers 16 tokens x 64 bytes.
template <int DT, bool QK>
__device__ __forceinline__ void proj_epilogue16(const ProjArgs &a, accv_t (&acc)[kNB][kTB], uint32_t m0,
                                                uint32_t hd, int wt, int lane, const float4 *tbl) {
    const uint32_t q = lane >> 4;
    const int comp = hd < a.Hq ? 0 : (hd < a.Hq + a.Hkv ? 1 : 2);
    const uint32_t hc = hd - (comp == 0 ? 0u : (comp == 1 ? a.Hq : a.Hq + a.Hkv));
    uint32_t qd, jd;
    a.hl[comp].divmod(hc, qd, jd);
    uint16_t *dbase = a.dst[comp] + int64_t(qd) * a.d_q[comp] + int64_t(jd) * kProjD;
    const int64_t d_b = a.d_b[comp], d_g = a.d_g[comp];

    // this lane's 32 norm weights, d = 16nb + 4q + 0..3, widened once
    float wf[kNB][4];
    if constexpr (QK) {
        const uint16_t *wn = a.wn[comp];
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
            const uint2 w4 = *(const uint2 *)(wn + nb * 16 + q * 4);
            wf[nb][0] = widen1<DT>(w4.x & 0xFFFFu);
            wf[nb][1] = widen1<DT>(w4.x >> 16);
            wf[nb][2] = widen1<DT>(w4.y & 0xFFFFu);
            wf[nb][3] = widen1<DT>(w4.y >> 16);
        }
    }

#pragma unroll
    for (int tb = 0; tb < kTB; ++tb) {
        const int tl = wt * kWaveT + tb * 16 + (lane & 15);   // token within the block tile
        const uint32_t tok = m0 + tl;
        const bool live = tok < a.M;
        uint32_t b;
        const uint32_t g = token_pos(a, live ? tok : a.M - 1, b);
        float inv = 1.f;
        if constexpr (QK) {
            float ss = 0.f;
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
                for (int r = 0; r < 4; ++r) ss = fmaf(acc[nb][tb][r], acc[nb][tb][r], ss);
            // eps > 0 keeps the argument normal: the bare reciprocal square root suffices
            inv = __builtin_amdgcn_rsqf(fmaf(sum_rows4(ss), a.inv_D, a.eps));
        }
        uint16_t *drow = dbase + int64_t(b) * d_b + int64_t(g) * d_g;
        const float4 *trow = tbl + tl * kTblRow;
#pragma unroll
        for (int nbp = 0; nbp < kNB / 2; ++nbp) {
            uint32_t X[2], Y[2];   // the run of head-dim blocks 2nbp (X) and 2nbp+1 (Y), two pairs each
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int nb = 2 * nbp + h;
                uint32_t pk[2];
                if constexpr (QK) {
                    // pairs j0 = 8nb + 2q and j0 + 1: chunk j0 / 2 of the row (explicit fmas)
                    const float4 cs = trow[4 * nb + q];
#pragma unroll
                    for (int p = 0; p < 2; ++p) {
                        const float cv = p ? cs.z : cs.x, sv = p ? cs.w : cs.y;
                        const float n0 = acc[nb][tb][2 * p] * inv * wf[nb][2 * p];
                        const float n1 = acc[nb][tb][2 * p + 1] * inv * wf[nb][2 * p + 1];
                        pk[p] = pack2<DT>(fmaf(n0, cv, -(n1 * sv)), fmaf(n0, sv, n1 * cv));
                    }
                } else {
#pragma unroll
                    for (int p = 0; p < 2; ++p) pk[p] = pack2<DT>(acc[nb][tb][2 * p], acc[nb][tb][2 * p + 1]);
                }
                (h ? Y : X)[0] = pk[0];
                (h ? Y : X)[1] = pk[1];
            }
            // By rows, X = [x0 x1 x2 x3] and Y = [y0 y1 y2 y3] (x_q: d 4q..4q+3 of
            // block 2nbp).  Swapping the halves gives [x0 x1 y0 y1], [x2 x3 y2 y3];
            // swapping odd rows of the first with even rows of the second gives
            // [x0 x2 y0 y2], [x1 x3 y1 y3]: row q holds 8 consecutive values of
            // block 2nbp + q/2 at offset 8(q%2), in X then Y.
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const auto r0 = __builtin_amdgcn_permlane32_swap(X[i], Y[i], false, false);
                const auto r1 = __builtin_amdgcn_permlane16_swap(r0[0], r0[1], false, false);
                X[i] = r1[0];
                Y[i] = r1[1];
            }
            if (live) stg16(drow + (2 * nbp + (q >> 1)) * 16 + (q & 1) * 8, make_uint4(X[0], X[1], Y[0], Y[1]));
        }
    }
}

// The occupancy is fixed by the LDS (one block per CU); saying so keeps the
// scheduler from trading latency hiding for an occupancy it cannot reach.
template <int DT, int BD>
__global__ __launch_bounds__(kProjThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd, kWavesPerSimd)))
void proj_kernel(ProjArgs a) {
    constexpr int kDepthB = BD;
    static_assert(kDepthB >= kDepthA, "B at least as deep as A");
    __shared__ uint4 lds[lds_slots(kDepthB)];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);    // wave-uniform, so per-head choices are scalar
    const int wn = wv / kWavesT;       // head of the block this wave computes
    const int wt = wv % kWavesT;       // token slice of the block this wave computes
    uint32_t tile, hb;
    proj_block(a, blockIdx.x, gridDim.x, tile, hb);
    const uint32_t m0 = tile * kProjTileT;
    const uint32_t head0 = hb * kProjHeads;
    const uint32_t last_row = a.NH * kProjD - 1;        // an odd head count leaves the last block half empty

    // Per lane: the global 16-byte chunk of the slot it fills in each of its
    // load instructions (the same for every stage; only k moves).  Rows past
    // M read row M-1, weight rows past the last head the last row; neither is
    // stored.  The host keeps N*K/8 and M*K/8 below 2^31.
    const uint4 *wq = reinterpret_cast<const uint4 *>(a.w), *xq = reinterpret_cast<const uint4 *>(a.x);
    const uint32_t K8 = a.K / 8;
    uint32_t offA[kInstA], offB[kInstB];
#pragma unroll
    for (int u = 0; u < kInstA; ++u) {
        const int slot = (wv * kInstA + u) * 64 + lane;
        const int row = slot / kChunks, c = (slot % kChunks) ^ swz_key(row);
        offA[u] = min(head0 * kProjD + uint32_t(row), last_row) * K8 + c;
    }
#pragma unroll
    for (int u = 0; u < kInstB; ++u) {
        const int slot = (wv * kInstB + u) * 64 + lane;
        const int row = slot / kChunks, c = (slot % kChunks) ^ swz_key(row);
        offB[u] = min(m0 + uint32_t(row), a.M - 1) * K8 + c;
    }
    // LDS byte addresses (wave-uniform): the ring base and this wave's first
    // slot in the A and the B region of a stage.
    const uint32_t ring = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_char *)(&lds[0]));
    const uint32_t wu = __builtin_amdgcn_readfirstlane(uint32_t(wv));
    const uint32_t wA = wu * kInstA * 64 * 16;
    const uint32_t wB = kDepthA * kSlotsA * 16 + wu * kInstB * 64 * 16;
    // Load instruction u: A rows (u < kInstA) of stage ka into A slot sa, or
    // B rows of stage kb into B slot sb.
    auto load_one = [&](int u, uint32_t ka, uint32_t sa, uint32_t kb, uint32_t sb) {
        if (u < kInstA) dma16(wq + offA[u] + ka * (kProjTileK / 8), ring + sa * kSlotsA * 16 + wA + u * 64 * 16);
        else dma16(xq + offB[u - kInstA] + kb * (kProjTileK / 8),
                   ring + sb * kSlotsB * 16 + wB + (u - kInstA) * 64 * 16);
    };

    accv_t acc[kNB][kTB];
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
        for (int tb = 0; tb < kTB; ++tb)
#pragma unroll
            for (int i = 0; i < kMf * kMf / 64; ++i) acc[nb][tb][i] = 0.f;

    const uint32_t KT = a.K / kProjTileK;              // >= 1: the host requires K % 64 == 0, K > 0
    constexpr int kPer = kInstA + kInstB;              // this wave's load instructions per stage
    // the stages ahead of the first: A's, then B's (the waits below count on this order)
#pragma unroll
    for (int p = 0; p + 1 < kDepthA; ++p)
#pragma unroll
        for (int u = 0; u < kInstA; ++u) load_one(u, min(uint32_t(p), KT - 1), p, 0, 0);
#pragma unroll
    for (int p = 0; p + 1 < kDepthB; ++p)
#pragma unroll
        for (int u = kInstA; u < kPer; ++u) load_one(u, 0, 0, min(uint32_t(p), KT - 1), p);
    // At the top of stage kt its A and B loads must have landed.  Every
    // iteration issues its A loads (stage + kDepthA - 1) before its B loads
    // (stage + kDepthB - 1), so the loads still allowed in flight are the
    // later iterations' ones: after B(kt), (kDepthB - 2) iterations' worth;
    // after A(kt), its own iteration's B loads and (kDepthA - 2) iterations'.
    constexpr int kWaitB = (kDepthB - 2) * kPer, kWaitA = kInstB + (kDepthA - 2) * kPer;
    constexpr int kWait = kWaitB < kWaitA ? kWaitB : kWaitA;
    const int fr = lane % kMf;         // fragment row (A) / column (B) of this lane
    const int fk = lane / kMf;         // which 8-wide part of a K step
    // Main loop, in a fixed instruction order.  Each K step issues its
    // products one by one, with one fragment read of the next K step after
    // each of the first kNB+kTB products and this wave's loads of the stages
    // ahead (A's, then B's) spread over the products of the first kLoadKs
    // steps.  The last K step of a stage is read before the next barrier and
    // multiplied after it, so its products cover the LDS reads that open the
    // next stage, and the loads go out right after the barrier.  The loads
    // are unconditional: past the last stage they load it again into a free
    // slot (in bounds), and the epilogue waits for them before it reuses the
    // rings.
    // (Left to the compiler, the reads of a step were issued after most of
    // the products that could cover them.)
    constexpr int KS = kProjTileK / kKStep;
    constexpr int kM = kNB * kTB;                                 // products per K step
    constexpr int kR = kNB + kTB;                                 // fragment reads per K step
    constexpr int kLoadKs = ULY_PROJ_LOAD_KS < KS ? ULY_PROJ_LOAD_KS : KS;
    constexpr int kLPer = (kPer + kLoadKs - 1) / kLoadKs;         // loads per loading step
    static_assert(kR <= kM && kLPer <= kM, "schedule shape");
    auto read_frag = [&](const uint4 *sa, const uint4 *sb, int ks, int r, uint4 (&fa)[kNB], uint4 (&fb)[kTB]) {
        const int c = ks * (kKStep / 8) + fk;
        if (r < kNB) fa[r] = sa[swz(wn * kProjD + r * kMf + fr, c)];
        else fb[r - kNB] = sb[swz(wt * kWaveT + (r - kNB) * kMf + fr, c)];
    };
#define ULY_SB() __builtin_amdgcn_sched_barrier(0)
    // Products of (fa, fb); reads of K step `rks` (if >= 0) into (na, nb);
    // loads lbase .. lbase+lcount-1 (A of stage ka into A slot za, B of
    // stage kb into B slot zb).
    auto kstep = [&](const uint4 (&fa)[kNB], const uint4 (&fb)[kTB], uint4 (&na)[kNB], uint4 (&nb)[kTB],
                     const uint4 *sa, const uint4 *sb, int rks, int lbase, int lcount, uint32_t ka, uint32_t za,
                     uint32_t kb, uint32_t zb) {
#pragma unroll
        for (int i = 0; i < kM; ++i) {
            acc[i / kTB][i % kTB] = mfma<DT>(fa[i / kTB], fb[i % kTB], acc[i / kTB][i % kTB]);
            ULY_SB();
            if (rks >= 0 && i < kR) {
                read_frag(sa, sb, rks, i, na, nb);
                ULY_SB();
            }
            if (lcount > 0) {
                const int l0 = (i * lcount) / kM, l1 = ((i + 1) * lcount) / kM;
                if (l1 != l0) {
                    load_one(lbase + l0, ka, za, kb, zb);
                    ULY_SB();
                }
            }
        }
    };
    uint4 fa[kNB], fb[kTB], ga[kNB], gb[kTB];
    for (uint32_t kt = 0; kt < KT; ++kt) {
        wait_vmcnt<kWait>();
        lds_barrier();
        const uint32_t ka = min(kt + kDepthA - 1, KT - 1), za = (kt + kDepthA - 1) % kDepthA;
        const uint32_t kb = min(kt + kDepthB - 1, KT - 1), zb = (kt + kDepthB - 1) % kDepthB;
        const uint4 *sa = lds + (kt % kDepthA) * kSlotsA, *sb = lds + kDepthA * kSlotsA + (kt % kDepthB) * kSlotsB;
        // multiply steps of this iteration: m = 0 is the carried last step of
        // the previous stage (none at kt = 0, where step 0 is read first)
#pragma unroll
        for (int m = 0; m < KS; ++m) {
            // step m reads K step m of this stage and multiplies the fragments
            // of the step before it: the carried one for m = 0.  Even steps
            // multiply (fa, fb) and read into (ga, gb), odd steps the reverse.
            const int lb = m * kLPer, lc = m < kLoadKs ? (kPer - lb < kLPer ? kPer - lb : kLPer) : 0;
            if (kt == 0 && m == 0) {
                // nothing carried into the first stage: read step 0 where step
                // 1 expects it and issue this step's loads on their own
#pragma unroll
                for (int r = 0; r < kR; ++r) read_frag(sa, sb, 0, r, ga, gb);
#pragma unroll
                for (int l = 0; l < lc; ++l) load_one(lb + l, ka, za, kb, zb);
                ULY_SB();
                continue;
            }
            if ((m & 1) == 0) kstep(fa, fb, ga, gb, sa, sb, m, lb, lc, ka, za, kb, zb);
            else kstep(ga, gb, fa, fb, sa, sb, m, lb, lc, ka, za, kb, zb);
        }
        // step KS-1 read into (fa, fb) if KS-1 is odd, else into (ga, gb):
        // keep it in (fa, fb) for the carry
        if ((KS & 1) == 1) {
#pragma unroll
            for (int i = 0; i < kNB; ++i) fa[i] = ga[i];
#pragma unroll
            for (int i = 0; i < kTB; ++i) fb[i] = gb[i];
        }
    }
    if (KT > 0) kstep(fa, fb, ga, gb, nullptr, nullptr, -1, 0, 0, 0, 0, 0, 0);
#undef ULY_SB
    wait_vmcnt<0>();      // the last stage's repeat loads land before the ring is reused

    // The ring is free once every wave is past its last stage: stage the
    // block's table rows there (only blocks with a q or k head rotate).
    float4 *tbl = reinterpret_cast<float4 *>(lds);
    lds_barrier();
    if (head0 < a.Hq + a.Hkv) {
        stage_table(a, m0, tbl, tid);
        lds_barrier();
    }
    const uint32_t hd = head0 + wn;
    if constexpr (kMf == 32) {
        if (hd < a.Hq + a.Hkv) proj_epilogue<DT, true>(a, acc, m0, hd, wt, lane, tbl);
        else if (hd < a.NH) proj_epilogue<DT, false>(a, acc, m0, hd, wt, lane, tbl);
    } else {
        if (hd < a.Hq + a.Hkv) proj_epilogue16<DT, true>(a, acc, m0, hd, wt, lane, tbl);
        else if (hd < a.NH) proj_epilogue16<DT, false>(a, acc, m0, hd, wt, lane, tbl);
    }
}

}  // namespace

#ifndef ULY_PROJ_DEEP_BD
#define ULY_PROJ_DEEP_BD 3
#endif
static_assert(lds_slots(ULY_PROJ_DEEP_BD) * 16 <= 160 * 1024, "LDS of one workgroup");

void launch_proj(const ProjArgs &a, int dtype, uint32_t blocks, bool deep_b, hipStream_t stream) {
    constexpr int kDeep = ULY_PROJ_DEEP_BD;      // token-row ring depth for operands streaming from HBM
    if (dtype == ULY_BF16) {
        if (deep_b) hipLaunchKernelGGL((proj_kernel<2, kDeep>), dim3(blocks), dim3(kProjThreads), 0, stream, a);
        else hipLaunchKernelGGL((proj_kernel<2, 2>), dim3(blocks), dim3(kProjThreads), 0, stream, a);
    } else {
        if (deep_b) hipLaunchKernelGGL((proj_kernel<1, kDeep>), dim3(blocks), dim3(kProjThreads), 0, stream, a);
        else hipLaunchKernelGGL((proj_kernel<1, 2>), dim3(blocks), dim3(kProjThreads), 0, stream, a);
    }
}

}  // namespace uly
