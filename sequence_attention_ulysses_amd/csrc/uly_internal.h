// Private declarations shared by the host runtime (uly_runtime.cpp) and the
// gfx950 kernels (uly_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "fastdiv.h"

namespace uly {

// ---------------------------------------------------------------------------
// Chunk relayout.  A Ulysses exchange moves contiguous chunks of Hl*D
// elements (one token's head band) between two 4-D index spaces.  A
// thread's flat 16-byte vector index i splits into 4 outer indices (i0
// outermost) and the vector position c inside the chunk,
//   i = (((i0*n1 + i1)*n2 + i2)*n3 + i3)*vpc + c
//   src = src_base + i0*ss[0] + i1*ss[1] + i2*ss[2] + i3*ss[3] + 16*c   (bytes)
//   dst = dst_base + i0*ds[0] + i1*ds[1] + i2*ds[2] + i3*ds[3] + 16*c
// The planner picks which side is dense in i.
// ---------------------------------------------------------------------------
struct CopyPlan {
    const uint8_t *src;
    uint8_t *dst;
    int64_t ss[4];
    int64_t ds[4];
    FastDiv vpc;         // 16-byte vectors per chunk
    FastDiv n3, n2, n1;  // extents of the inner three outer dims
    uint32_t total;      // vectors in this plan
    uint32_t first_block;
};

constexpr int kMaxPlans = 3;

struct CopyBatch {
    CopyPlan p[kMaxPlans];
    int n;
    uint32_t blocks;
};

// ---------------------------------------------------------------------------
// Fused RMSNorm + RoPE + scatter.  Rows are (r, b, s, hh) in source order,
// hh in [0, H0 + H1 + H2): hh < H0 reads operand 0 (Q), hh < H0 + H1
// operand 1 (K), the rest operand 2 (V, copied unchanged), so the rows of
// one token share one table row.
// ---------------------------------------------------------------------------
struct NormRopeOperand {
    const uint16_t *src;
    uint16_t *dst;
    const uint16_t *w;
    int64_t s_rank, s_b, s_s, s_h;   // source element strides
    int64_t d_q, d_b, d_g, d_j;      // destination element strides (rank, batch, global token, head)
    FastDiv hl;                      // heads per rank
    uint32_t H;
    uint32_t pad;
};

struct NormRopeArgs {
    NormRopeOperand op[3];
    const float *cos_tab;
    const float *sin_tab;
    FastDiv rpt;        // rows per token = H0 + H1 + H2
    FastDiv sl;         // S_l
    FastDiv bdiv;       // B
    uint32_t H0;        // rows of operand 0 per token (0 when absent)
    uint32_t H01;       // H0 + H1
    uint32_t tokens;    // P*B*S_l
    uint32_t S_l;
    uint32_t D;
    float eps;
    float inv_D;
    // operand-major band form: block row k of the grid's operand-major order
    // belongs to operand task_op[k] (the operands present, in order)
    uint32_t P;
    uint32_t task_op[3];
};

// ---------------------------------------------------------------------------
// Row maps with zero fill: sequence pad/trim and the spatial height shards.
// Each destination row of `vpr` 16-byte vectors is copied from one source
// row or zero-filled.
// ---------------------------------------------------------------------------
enum RowMapKind : int {
    kPadShard = 0,       // dst x[P][B][S_l] rows  <- full[B][S] rows, zero past S
    kUnshardTrim = 1,    // dst full[B][S] rows    <- x[P][B][S_l] rows
    kSplitHalo = 2,      // dst sh[P][N][hmax+2h]  <- full[N][Hh], zero outside
    kGatherStacked = 3,  // dst st[P][N][hmax]     <- sh[P][N][hmax+2h] core rows
    kTrimConcat = 4      // dst full[N][Hh]        <- st[P][N][hmax]
};

struct RowMapArgs {
    const uint8_t *src;
    uint8_t *dst;
    FastDiv vpr;         // 16-byte vectors per row
    FastDiv f0;          // innermost destination row dimension
    FastDiv f1;          // next destination row dimension
    FastDiv f2;          // mode-specific: S_l (unshard) or base_h + 1 (trim/concat)
    FastDiv f3;          // mode-specific: base_h (trim/concat)
    uint32_t total;      // vectors written
    uint32_t B_or_N;     // batch (pad/trim) or flattened leading dims N (spatial)
    uint32_t S;          // pad/trim: real sequence length; spatial: Hh
    uint32_t S_l;        // pad/trim: rows per rank; spatial: hmax
    uint32_t halo;
    uint32_t base_h;     // spatial: floor(Hh / P)
    uint32_t extra_h;    // spatial: Hh % P
    uint32_t pad;
};

// Launch wrappers (uly_kernels.hip).  They only enqueue; the caller checks
// hipGetLastError().
void launch_relayout(const CopyBatch &b, hipStream_t stream);
void launch_norm_rope(const NormRopeArgs &a, int lanes, int dtype, bool uniform, bool tile, uint32_t blocks,
                      hipStream_t stream);
void launch_norm_rope_band(const NormRopeArgs &a, int dtype, uint32_t blocks, hipStream_t stream);
void launch_rowmap(const RowMapArgs &a, int kind, hipStream_t stream);

#ifndef ULY_THREADS
#define ULY_THREADS 256
#endif
#ifndef ULY_COPY_UNROLL
#define ULY_COPY_UNROLL 1
#endif
#ifndef ULY_ROPE_TOKENS
#define ULY_ROPE_TOKENS 2
#endif
#ifndef ULY_ROPE_SLOTS
#define ULY_ROPE_SLOTS 1
#endif
#ifndef ULY_ROPE_THREADS
#define ULY_ROPE_THREADS 768
#endif
#ifndef ULY_BAND_WAVES
#define ULY_BAND_WAVES 4
#endif
#ifndef ULY_BAND_TOKENS
#define ULY_BAND_TOKENS 2
#endif
#ifndef ULY_BAND_INFLIGHT
#define ULY_BAND_INFLIGHT 5
#endif
#ifndef ULY_RELAYOUT_NT_LOAD
#define ULY_RELAYOUT_NT_LOAD 1
#endif
#ifndef ULY_RELAYOUT_NT_STORE
#define ULY_RELAYOUT_NT_STORE 1
#endif
#ifndef ULY_EXCHANGE_LOAD
#define ULY_EXCHANGE_LOAD 1
#endif
#ifndef ULY_EXCHANGE_STORE
#define ULY_EXCHANGE_STORE 2
#endif
#ifndef ULY_ROPE_NT_LOAD
#define ULY_ROPE_NT_LOAD 1
#endif
#ifndef ULY_ROPE_NT_STORE
#define ULY_ROPE_NT_STORE 1
#endif
// Cache policy of the operand loads and stores per kernel: 0 ordinary,
// 1 non-temporal (streaming), 2 system scope.
constexpr int kRelayoutNtLoad = ULY_RELAYOUT_NT_LOAD;     // row maps (pad/trim, spatial)
constexpr int kRelayoutNtStore = ULY_RELAYOUT_NT_STORE;
constexpr int kExchangeLoad = ULY_EXCHANGE_LOAD;           // scatter, gather and chunk exchange
constexpr int kExchangeStore = ULY_EXCHANGE_STORE;
// Operands beyond the 256 MB Infinity Cache stream from HBM (the projection
// picks its deeper token ring for them).
constexpr int64_t kCacheResidentBytes = int64_t(256) << 20;
constexpr int kRopeNtLoad = ULY_ROPE_NT_LOAD;
constexpr int kRopeNtStore = ULY_ROPE_NT_STORE;
constexpr int kThreads = ULY_THREADS;
constexpr int kCopyUnroll = ULY_COPY_UNROLL;             // 16-byte vectors per thread
constexpr uint32_t kCopyVecsPerBlock = kThreads * kCopyUnroll;
constexpr int kRopeTokens = ULY_ROPE_TOKENS;            // tokens per block
constexpr int kRopeSlots = ULY_ROPE_SLOTS;              // head slots a lane group loads at once
constexpr int kRopeThreads = ULY_ROPE_THREADS;          // threads per block of the fused kernel
constexpr int kBandWaves = ULY_BAND_WAVES;              // waves per block of the operand-major band form
constexpr int kBandTokens = ULY_BAND_TOKENS;            // tokens per block there
constexpr int kBandInflight = ULY_BAND_INFLIGHT;        // row loads a lane keeps in flight there

}  // namespace uly
