// gfx950 kernels of the Ulysses exchange (one GPU, P rank slabs in HBM).
//
// Every kernel here is bound by HBM bandwidth: the relayouts are pure
// permutations of contiguous chunks, and the fused norm + RoPE does ~10 fp32
// operations per 4 bytes moved.  The design therefore aims at bytes in
// flight and full 16-byte accesses, not at arithmetic:
//   * every lane moves 16-byte vectors (global_load/store_dwordx4), a wave
//     moves 1 KiB contiguous runs of the destination;
//   * a thread issues all of its loads before any store so several vectors
//     per lane are in flight;
//   * no LDS: the exchange permutes whole head-band chunks (>= 256 bytes),
//     so both the source and the destination side of every wave access are
//     already contiguous and coalesced.  Staging a block's rows through an
//     LDS tile to store each (operand, destination band) as one 3-12 KiB run
//     was measured on the fused kernel: 113-119 us against 104 us at the
//     video-DiT shape, since a block's stores then wait behind its loads
//     instead of streaming beside them;
//   * no MFMA: there is no contraction on this path.
//
// Pages cited (by title and section): TeleFuser documentation,
// "Communication Architecture" ("Ulysses", "Equal-shape gather", "Spatial
// VAE Communication"); flashinfer PR #6332 ("Description", "Assumptions").

#include <hip/hip_runtime.h>

#include "uly_internal.h"

namespace uly {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) u32x4 global_u32x4;

// All operands live in device (global) memory: the explicit address space
// keeps the accesses global_load/store instead of flat ones.  Operand data
// streams through exactly once; each kernel picks the cache policy of its
// loads and of its stores (uly_internal.h).  Measured with steps run back to
// back over rotating buffer sets (so every byte a step writes is charged to
// the steps): the exchange kernels (scatter, gather, chunk exchange) run
// fastest with non-temporal loads and system-scope stores (video-DiT output
// gather 37.1 -> 32.8 us, GQA Q/K/V scatter 525 -> 506 us against
// non-temporal or system-scope accesses on both sides), the fused norm + RoPE
// kernels with non-temporal loads and stores (ordinary or system-scope
// stores finish the fused launch sooner, 98 us against 104, but leave
// write-back that the next launch pays for: step 150-155 us against 139).
// Policy 0: ordinary access; 1: non-temporal (nt); 2: system scope (sc0 sc1,
// through a volatile access).
template <int POL>
__device__ __forceinline__ uint4 load16(const void *p) {
    const global_u32x4 *g = (const global_u32x4 *)p;
    u32x4 v;
    if constexpr (POL == 1) v = __builtin_nontemporal_load(g);
    else if constexpr (POL == 2) v = *(const volatile global_u32x4 *)g;
    else v = *g;
    return make_uint4(v.x, v.y, v.z, v.w);
}

template <int POL>
__device__ __forceinline__ void store16(void *p, uint4 v) {
    global_u32x4 *g = (global_u32x4 *)p;
    const u32x4 w = {v.x, v.y, v.z, v.w};
    if constexpr (POL == 1) __builtin_nontemporal_store(w, g);
    else if constexpr (POL == 2) *(volatile global_u32x4 *)g = w;
    else *g = w;
}

// Data every block re-reads (norm weights): ordinary cached load.
__device__ __forceinline__ uint4 load16_cached(const void *p) {
    const u32x4 v = *(const global_u32x4 *)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Table rows are re-read by every head of a token: ordinary cached loads.
__device__ __forceinline__ float4 load_table4(const float *p) {
    const global_u32x4 *g = (const global_u32x4 *)p;
    const u32x4 v = *g;
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}

// Blocks are dispatched to the 8 XCDs of the chip round-robin.  With
// ULY_XCD_REMAP the logical block index is permuted so that XCD x works
// through one contiguous range of the grid (a bijection for any grid size).
__device__ __forceinline__ uint32_t logical_block(uint32_t bid, uint32_t grid) {
#ifdef ULY_XCD_REMAP
    constexpr uint32_t kXcds = 8;
    const uint32_t q = grid / kXcds, r = grid % kXcds;
    const uint32_t x = bid % kXcds, k = bid / kXcds;
    return x * q + min(x, r) + k;
#else
    (void)grid;
    return bid;
#endif
}

// ---------------------------------------------------------------------------
// Chunk relayout (Ulysses scatter and gather, "Communication Architecture",
// "Ulysses").  Up to three operands (Q, K, V) share one launch: blocks
// [p[i].first_block, p[i+1].first_block) belong to operand i, so the three
// copies fill the machine together instead of draining one after another.
// ---------------------------------------------------------------------------
template <int LP, int SP>
__global__ __launch_bounds__(kThreads) void relayout_kernel(CopyBatch b) {
    const uint32_t bid = logical_block(blockIdx.x, gridDim.x);
    int pi = 0;
    if (b.n > 1 && bid >= b.p[1].first_block) pi = 1;
    if (b.n > 2 && bid >= b.p[2].first_block) pi = 2;
    const CopyPlan &P = b.p[pi];

    const uint32_t first = (bid - P.first_block) * kCopyVecsPerBlock + threadIdx.x;
    uint4 v[kCopyUnroll];
    uint8_t *d[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const uint32_t i = first + u * kThreads;
        if (i < P.total) {
            uint32_t t, c, i0, i1, i2, i3;
            P.vpc.divmod(i, t, c);
            P.n3.divmod(t, t, i3);
            P.n2.divmod(t, t, i2);
            P.n1.divmod(t, i0, i1);
            const uint8_t *s = P.src + int64_t(i0) * P.ss[0] + int64_t(i1) * P.ss[1] +
                               int64_t(i2) * P.ss[2] + int64_t(i3) * P.ss[3] + uint64_t(c) * 16u;
            d[u] = P.dst + int64_t(i0) * P.ds[0] + int64_t(i1) * P.ds[1] + int64_t(i2) * P.ds[2] +
                   int64_t(i3) * P.ds[3] + uint64_t(c) * 16u;
            v[u] = load16<LP>(s);
        }
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const uint32_t i = first + u * kThreads;
        if (i < P.total) store16<SP>(d[u], v[u]);
    }
}

// ---------------------------------------------------------------------------
// Fused per-head RMSNorm + interleaved RoPE + Ulysses scatter (flashinfer
// PR #6332, "Assumptions"): one row of D values is spread over LANES lanes
// of 8 values (16 bytes) each, so a D = 128 16-bit row is 16 lanes — one
// DPP row of the wavefront.  The sum of squares is reduced with DPP moves
// inside that row, the interleaved pairs (2j, 2j+1) of a lane are rotated
// in registers (a pair never straddles lanes), and the result is rounded
// once to 16 bits and stored at the row's head-sharded destination.
// ---------------------------------------------------------------------------
template <int LANES>
__device__ __forceinline__ float row_sum(float v) {
    // quad_perm [1,0,3,2] and [2,3,0,1]: sums over 4 lanes
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
    if constexpr (LANES >= 8)   // row_half_mirror: lane i <-> 7-i within 8 lanes
        v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
    if constexpr (LANES >= 16)  // row_mirror: lane i <-> 15-i within 16 lanes
        v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));
    if constexpr (LANES >= 32)  // across the two 16-lane rows of a 32-lane group
        v += __shfl_xor(v, 16, 64);
    return v;
}

template <int DT>
__device__ __forceinline__ void unpack8(uint4 raw, float (&x)[8]) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (DT == 2) {  // bf16: the high half of an fp32
            x[2 * i] = __uint_as_float(w[i] << 16);
            x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        } else {                  // fp16
            _Float16 lo = __builtin_bit_cast(_Float16, uint16_t(w[i] & 0xFFFFu));
            _Float16 hi = __builtin_bit_cast(_Float16, uint16_t(w[i] >> 16));
            x[2 * i] = float(lo);
            x[2 * i + 1] = float(hi);
        }
    }
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    // v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32: round to nearest even
    if constexpr (DT == 2) {
        bf16x2_t p = {__bf16(a), __bf16(b)};
        return __builtin_bit_cast(uint32_t, p);
    } else {
        f16x2_t p = {_Float16(a), _Float16(b)};
        return __builtin_bit_cast(uint32_t, p);
    }
}

template <class T>
__device__ __forceinline__ T sel3(uint32_t i, T a, T b, T c) {
    return i == 0 ? a : (i == 1 ? b : c);
}

// One lane's eight values of a row: RMSNorm with its weights, then the
// rotation of the lane's four interleaved pairs, each result rounded once to
// 16 bits.  The rotation's products are combined in explicit fused
// multiply-adds, y0 = fma(n0, c, -(n1 s)) and y1 = fma(n0, s, n1 c), so every
// kernel that calls this rounds the same way whichever products the compiler
// would otherwise have contracted.  The row's sum of squares comes in `ss`.
template <int DT>
__device__ __forceinline__ uint4 norm_rope8(const float (&x)[8], float ss, const float (&w)[8], float4 c4, float4 s4,
                                            float inv_D, float eps) {
    // eps > 0 keeps the argument normal: the bare reciprocal square root suffices
    const float inv = __builtin_amdgcn_rsqf(fmaf(ss, inv_D, eps));
    const float c[4] = {c4.x, c4.y, c4.z, c4.w};
    const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
    uint32_t out[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const float n0 = (x[2 * p] * inv) * w[2 * p];
        const float n1 = (x[2 * p + 1] * inv) * w[2 * p + 1];
        out[p] = pack2<DT>(fmaf(n0, c[p], -(n1 * sv[p])), fmaf(n0, sv[p], n1 * c[p]));
    }
    return make_uint4(out[0], out[1], out[2], out[3]);
}

// Work mapping.  A block owns a tile of kRopeTokens consecutive tokens
// (source order r, b, s).  Its GROUPS lane groups split the R = H0+H1+H2
// rows of a token: group gi owns the row slots hh = gi, gi + GROUPS, ...,
// the same for every token, so the per-head part of the addressing is
// computed once per slot, and the token part (r, b, s, g and the token
// offsets) is the same for every lane of the block and lives in scalar
// registers.
//   UNI:  every operand's head count is a multiple of the groups per wave,
//         so a wave's slots never straddle two operands: the operand of a
//         slot is wave-uniform and every per-operand field is a scalar.
//   TILE: S_l is a multiple of the tile, so a tile never crosses a rank or
//         batch boundary: one decode per block, token t of the tile is
//         s0 + t at global position g0 + t, and there is no partial tile.
// Rows of operand 2 (V) ride in the same grid as plain 16-byte copies: the
// whole Q/K/V scatter is one launch that shares HBM bandwidth without a
// second kernel's ramp-up and tail.
#ifdef ULY_ROPE_WAVES_PER_EU
#define ULY_ROPE_OCCUPANCY __attribute__((amdgpu_waves_per_eu(ULY_ROPE_WAVES_PER_EU)))
#else
#define ULY_ROPE_OCCUPANCY
#endif

// One head slot of a lane group: where its rows come from and go to.
struct Slot {
    const uint16_t *src;   // this lane's 8 elements of the head, token offsets still to add
    uint16_t *dst;
    const uint16_t *w;     // this lane's 8 norm weights (V: any readable 16 bytes, unused)
    int64_t s_rank, s_b, s_s, d_b, d_g;
    bool rope;             // Q or K (normalised and rotated); V is copied
    bool live;             // the slot exists (the last slots of a group may not)
};

// Addresses only: the loads are issued by the caller, rows first, so that
// no load result is consumed before every load of the trip is in flight.
template <bool UNI>
__device__ __forceinline__ Slot make_slot(const NormRopeArgs &a, uint32_t hh, uint32_t R, uint32_t lane) {
    const NormRopeOperand &o0 = a.op[0], &o1 = a.op[1], &o2 = a.op[2];
    Slot sl;
    sl.live = hh < R;
    const uint32_t hc = sl.live ? hh : R - 1;                  // dead slots read a valid row
    const uint32_t hh_op = UNI ? __builtin_amdgcn_readfirstlane(hc) : hc;
    const uint32_t oi = (hh_op >= a.H0 ? 1u : 0u) + (hh_op >= a.H01 ? 1u : 0u);
    const uint32_t h = hc - sel3(oi, 0u, a.H0, a.H01);
    uint32_t qd, j;
    if constexpr (UNI) {
        // the operand is wave-uniform: read its fields alone, from the
        // kernel arguments at a scalar index (selecting each field among all
        // three kept every operand's fields live and spilled 16 SGPRs)
        const NormRopeOperand &o = a.op[oi];
        o.hl.divmod(h, qd, j);
        sl.s_rank = o.s_rank;
        sl.s_b = o.s_b;
        sl.s_s = o.s_s;
        sl.d_b = o.d_b;
        sl.d_g = o.d_g;
        sl.src = o.src + int64_t(h) * o.s_h + lane * 8;
        sl.dst = o.dst + int64_t(qd) * o.d_q + int64_t(j) * o.d_j + lane * 8;
        sl.w = o.w + lane * 8;
        sl.rope = oi < 2;
        return sl;
    }
    // per lane: select each field among the three operands
    if (oi == 0) o0.hl.divmod(h, qd, j);
    else if (oi == 1) o1.hl.divmod(h, qd, j);
    else o2.hl.divmod(h, qd, j);
    sl.s_rank = sel3(oi, o0.s_rank, o1.s_rank, o2.s_rank);
    sl.s_b = sel3(oi, o0.s_b, o1.s_b, o2.s_b);
    sl.s_s = sel3(oi, o0.s_s, o1.s_s, o2.s_s);
    sl.d_b = sel3(oi, o0.d_b, o1.d_b, o2.d_b);
    sl.d_g = sel3(oi, o0.d_g, o1.d_g, o2.d_g);
    sl.src = sel3(oi, o0.src, o1.src, o2.src) + int64_t(h) * sel3(oi, o0.s_h, o1.s_h, o2.s_h) + lane * 8;
    sl.dst = sel3(oi, o0.dst, o1.dst, o2.dst) + int64_t(qd) * sel3(oi, o0.d_q, o1.d_q, o2.d_q) +
             int64_t(j) * sel3(oi, o0.d_j, o1.d_j, o2.d_j) + lane * 8;
    sl.w = sel3(oi, o0.w, o1.w, o2.w) + lane * 8;
    sl.rope = oi < 2;
    return sl;
}

// Work mapping.  A block owns a tile of kRopeTokens consecutive tokens
// (source order r, b, s).  Its GROUPS lane groups split the R = H0+H1+H2
// rows of a token: group gi owns the row slots hh = gi, gi + GROUPS, ...,
// the same for every token, and loads kRopeSlots of them at once.  The
// per-head part of the addressing is computed once per slot; the token
// part (r, b, s, g, the table row) once per block.
//   UNI:  every operand's head count is a multiple of the groups per wave,
//         so a wave's slots never straddle two operands: the operand of a
//         slot is wave-uniform and every per-operand field is a scalar.
//   TILE: S_l is a multiple of the tile, so a tile never crosses a rank or
//         batch boundary: one decode per block, token t of the tile is
//         s0 + t at global position g0 + t, and there is no partial tile.
// Rows of operand 2 (V) ride in the same grid as plain 16-byte copies: the
// whole Q/K/V scatter is one launch that shares HBM bandwidth without a
// second kernel's ramp-up and tail.
template <int LANES, int DT, bool UNI, bool TILE>
__global__ __launch_bounds__(kRopeThreads) ULY_ROPE_OCCUPANCY void norm_rope_kernel(NormRopeArgs a) {
    constexpr int GROUPS = kRopeThreads / LANES;
    constexpr int TU = kRopeTokens;
    constexpr int SU = kRopeSlots;
    const uint32_t lane = threadIdx.x % LANES;
    const uint32_t grp = threadIdx.x / LANES;
    const uint32_t half = a.D / 2;
    const uint32_t R = a.rpt.d;
    const uint32_t tk0 = logical_block(blockIdx.x, gridDim.x) * TU;

    // Token part, once per block: (r, b, s, g) of each token and its table row.
    uint32_t tr[TU], tb[TU], ts[TU];
    bool live[TU];
    float4 cs[TU], sn[TU];
#pragma unroll
    for (int t = 0; t < TU; ++t) {
        uint32_t rb, g;
        if (TILE) {
            if (t == 0) {
                a.sl.divmod(tk0, rb, ts[0]);
                a.bdiv.divmod(rb, tr[0], tb[0]);
            } else {
                tr[t] = tr[0];
                tb[t] = tb[0];
                ts[t] = ts[0] + t;
            }
            live[t] = true;
        } else {
            live[t] = tk0 + t < a.tokens;          // uniform across the block
            const uint32_t tk = live[t] ? tk0 + t : a.tokens - 1;
            a.sl.divmod(tk, rb, ts[t]);
            a.bdiv.divmod(rb, tr[t], tb[t]);
        }
        g = tr[t] * a.S_l + ts[t];
        // unconditional: the table covers every position (a V-only call reads
        // and ignores it), and a load under a branch would be waited for at once
        const size_t t_off = size_t(g) * half + lane * 4;
        cs[t] = load_table4(a.cos_tab + t_off);
        sn[t] = load_table4(a.sin_tab + t_off);
    }

    // Every lane of a group runs the same slot and token trips; dead slots
    // and tokens past the end are computed on a valid row and not stored, so
    // every lane of a group takes part in every DPP exchange.
    for (uint32_t hh = grp; hh < R; hh += GROUPS * SU) {
        Slot sl[SU];
        uint4 raw[SU][TU], wraw[SU];
#pragma unroll
        for (int u = 0; u < SU; ++u) sl[u] = make_slot<UNI>(a, hh + u * GROUPS, R, lane);
        // every row load of the trip first, then the (cache-resident) weights
#pragma unroll
        for (int u = 0; u < SU; ++u)
#pragma unroll
            for (int t = 0; t < TU; ++t)
                raw[u][t] = load16<kRopeNtLoad>(sl[u].src + (int64_t(tr[t]) * sl[u].s_rank + int64_t(tb[t]) * sl[u].s_b +
                                                int64_t(ts[t]) * sl[u].s_s));
#pragma unroll
        for (int u = 0; u < SU; ++u) wraw[u] = load16_cached(sl[u].w);
#pragma unroll
        for (int u = 0; u < SU; ++u) {
            if (UNI && !sl[u].rope) {
                // a V slot (wave-uniform here): the rows are stored as loaded,
                // without the discarded norm and rotation (0.5 % of the step)
#pragma unroll
                for (int t = 0; t < TU; ++t) {
                    const uint32_t g = tr[t] * a.S_l + ts[t];
                    if (sl[u].live && live[t])
                        store16<kRopeNtStore>(sl[u].dst + (int64_t(tb[t]) * sl[u].d_b + int64_t(g) * sl[u].d_g),
                                              raw[u][t]);
                }
                continue;
            }
            float w[8];
            unpack8<DT>(wraw[u], w);
#pragma unroll
            for (int t = 0; t < TU; ++t) {
                float x[8];
                unpack8<DT>(raw[u][t], x);
                float ss = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) ss = fmaf(x[i], x[i], ss);
                ss = row_sum<LANES>(ss);
                const uint4 rot = norm_rope8<DT>(x, ss, w, cs[t], sn[t], a.inv_D, a.eps);
                const uint4 res = sl[u].rope ? rot : raw[u][t];
                const uint32_t g = tr[t] * a.S_l + ts[t];
                if (sl[u].live && live[t])
                    store16<kRopeNtStore>(sl[u].dst + (int64_t(tb[t]) * sl[u].d_b + int64_t(g) * sl[u].d_g), res);
            }
        }
    }
}

// Operand-major band form, for operands that are each one dense tensor
// (Q, K and V not interleaved in a fused projection).  A block owns one
// operand of a tile of kBandTokens consecutive tokens of one rank and batch
// (S_l a multiple of the tile); the grid runs operand by operand, so the
// blocks in flight read one operand's tensor front to back and write only
// its P destination bands.  Each wave owns one destination rank q at a time:
// the Hl head rows of band q for every token of the tile, which are one
// contiguous run of the destination (Hl * tokens * D elements).  The wave
// walks the run four rows at a time (one per 16-lane group), so every store
// instruction writes 1 KiB of consecutive destination bytes.  D = 128
// (16 lanes per row).  V blocks store their rows as loaded; the runtime
// hands this kernel V only for the packed receive layout, and moves a V
// with a target of its own by the relayout kernel, which copies dense
// operands at the plain copy rate.
template <int DT>
__global__ __launch_bounds__(kBandWaves * 64) void norm_rope_band_kernel(NormRopeArgs a) {
    constexpr int LANES = 16, GPW = 64 / LANES, TU = kBandTokens, MAXT = kBandInflight;
    const uint32_t lane = threadIdx.x % LANES;
    const uint32_t gi = (threadIdx.x % 64) / LANES;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const uint32_t ntiles = a.tokens / TU;
    const uint32_t lb = logical_block(blockIdx.x, gridDim.x);
    const uint32_t op_slot = lb / ntiles;                    // block-uniform
    const uint32_t tk0 = (lb - op_slot * ntiles) * TU;
    const uint32_t oi = sel3(op_slot, a.task_op[0], a.task_op[1], a.task_op[2]);
    uint32_t rb, s0, r, b;
    a.sl.divmod(tk0, rb, s0);
    a.bdiv.divmod(rb, r, b);
    const uint32_t g0 = r * a.S_l + s0;
    // this lane's cos/sin of every token of the tile
    float4 cs[TU], sn[TU];
    const bool rope = oi < 2;                                // a V block rotates nothing: no table row
#pragma unroll
    for (int t = 0; t < TU; ++t) {
        const size_t t_off = size_t(g0 + t) * (a.D / 2) + lane * 4;
        cs[t] = rope ? load_table4(a.cos_tab + t_off) : make_float4(1.f, 1.f, 1.f, 1.f);
        sn[t] = rope ? load_table4(a.sin_tab + t_off) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    for (uint32_t q = wave; q < a.P; q += kBandWaves) {
        const NormRopeOperand &o0 = a.op[0], &o1 = a.op[1], &o2 = a.op[2];
        const FastDiv hl = oi == 0 ? o0.hl : (oi == 1 ? o1.hl : o2.hl);
        const uint32_t Hl = hl.d;
        const uint32_t rows = Hl * TU;
        const int64_t s_s = sel3(oi, o0.s_s, o1.s_s, o2.s_s), s_h = sel3(oi, o0.s_h, o1.s_h, o2.s_h);
        const int64_t d_g = sel3(oi, o0.d_g, o1.d_g, o2.d_g), d_j = sel3(oi, o0.d_j, o1.d_j, o2.d_j);
        const uint16_t *src = sel3(oi, o0.src, o1.src, o2.src) + int64_t(r) * sel3(oi, o0.s_rank, o1.s_rank, o2.s_rank) +
                              int64_t(b) * sel3(oi, o0.s_b, o1.s_b, o2.s_b) + int64_t(s0) * s_s +
                              int64_t(q) * Hl * s_h + lane * 8;
        uint16_t *dst = sel3(oi, o0.dst, o1.dst, o2.dst) + int64_t(q) * sel3(oi, o0.d_q, o1.d_q, o2.d_q) +
                        int64_t(b) * sel3(oi, o0.d_b, o1.d_b, o2.d_b) + int64_t(g0) * d_g + lane * 8;
        const uint4 wraw = load16_cached(sel3(oi, o0.w, o1.w, o2.w) + lane * 8);
        for (uint32_t k0 = 0; k0 < rows; k0 += GPW * MAXT) {
            uint4 raw[MAXT];
            uint32_t tt[MAXT], jj[MAXT];
#pragma unroll
            for (int u = 0; u < MAXT; ++u) {
                const uint32_t k = min(k0 + u * GPW + gi, rows - 1);
                hl.divmod(k, tt[u], jj[u]);
                raw[u] = load16<kRopeNtLoad>(src + int64_t(tt[u]) * s_s + int64_t(jj[u]) * s_h);
            }
            if (!rope) {                                     // a V block (block-uniform): rows as loaded
#pragma unroll
                for (int u = 0; u < MAXT; ++u)
                    if (k0 + u * GPW + gi < rows)
                        store16<kRopeNtStore>(dst + int64_t(tt[u]) * d_g + int64_t(jj[u]) * d_j, raw[u]);
                continue;
            }
            float w[8];
            unpack8<DT>(wraw, w);
#pragma unroll
            for (int u = 0; u < MAXT; ++u) {
                const uint32_t k = k0 + u * GPW + gi;
                float x[8];
                unpack8<DT>(raw[u], x);
                float ss = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) ss = fmaf(x[i], x[i], ss);
                ss = row_sum<LANES>(ss);
                float4 c4 = cs[0], s4 = sn[0];
#pragma unroll
                for (int t = 1; t < TU; ++t)
                    if (tt[u] == uint32_t(t)) { c4 = cs[t]; s4 = sn[t]; }
                const uint4 rot = norm_rope8<DT>(x, ss, w, c4, s4, a.inv_D, a.eps);
                if (k < rows)
                    store16<kRopeNtStore>(dst + int64_t(tt[u]) * d_g + int64_t(jj[u]) * d_j, rot);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Row maps with zero fill: sequence pad/trim (parallel_shard.py's role in
// "Communication Architecture") and height shards with halos, the
// rank-major stacked gather and its trim/concat ("Spatial VAE
// Communication", "Equal-shape gather").
// ---------------------------------------------------------------------------
template <int KIND>
__device__ __forceinline__ int64_t rowmap_source(const RowMapArgs &a, uint32_t row) {
    if constexpr (KIND == kPadShard) {
        uint32_t t, s, r, b;
        a.f0.divmod(row, t, s);
        a.f1.divmod(t, r, b);
        const uint32_t g = r * a.S_l + s;
        return g < a.S ? int64_t(b) * a.S + g : -1;
    } else if constexpr (KIND == kUnshardTrim) {
        uint32_t b, g, r, s;
        a.f0.divmod(row, b, g);
        a.f2.divmod(g, r, s);
        return (int64_t(r) * a.B_or_N + b) * a.S_l + s;
    } else if constexpr (KIND == kSplitHalo) {
        uint32_t t, i, r, n;
        a.f0.divmod(row, t, i);
        a.f1.divmod(t, r, n);
        const uint32_t h_r = a.base_h + (r < a.extra_h ? 1u : 0u);
        const int64_t o_r = int64_t(r) * a.base_h + min(r, a.extra_h);
        const int64_t sr = o_r - int64_t(a.halo) + i;
        if (i >= h_r + 2 * a.halo || sr < 0 || sr >= int64_t(a.S)) return -1;
        return int64_t(n) * a.S + sr;
    } else if constexpr (KIND == kGatherStacked) {
        uint32_t t, i, r, n;
        a.f0.divmod(row, t, i);
        a.f1.divmod(t, r, n);
        const uint32_t h_r = a.base_h + (r < a.extra_h ? 1u : 0u);
        if (i >= h_r) return -1;
        return (int64_t(r) * a.B_or_N + n) * (a.S_l + 2 * a.halo) + a.halo + i;
    } else {  // kTrimConcat
        uint32_t n, y, r, i;
        a.f0.divmod(row, n, y);
        const uint32_t boundary = a.extra_h * (a.base_h + 1);
        if (y < boundary) {
            a.f2.divmod(y, r, i);
        } else {
            a.f3.divmod(y - boundary, r, i);
            r += a.extra_h;
        }
        return (int64_t(r) * a.B_or_N + n) * a.S_l + i;
    }
}

template <int KIND>
__global__ __launch_bounds__(kThreads) void rowmap_kernel(RowMapArgs a) {
    const uint32_t first = blockIdx.x * kCopyVecsPerBlock + threadIdx.x;
    uint4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const uint32_t i = first + u * kThreads;
        v[u] = make_uint4(0, 0, 0, 0);
        if (i < a.total) {
            uint32_t row, c;
            a.vpr.divmod(i, row, c);
            const int64_t src_row = rowmap_source<KIND>(a, row);
            if (src_row >= 0) v[u] = load16<kRelayoutNtLoad>(a.src + (src_row * a.vpr.d + c) * 16);
        }
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const uint32_t i = first + u * kThreads;
        if (i < a.total) store16<kRelayoutNtStore>(a.dst + uint64_t(i) * 16u, v[u]);
    }
}

}  // namespace

void launch_relayout(const CopyBatch &b, hipStream_t stream) {
    hipLaunchKernelGGL((relayout_kernel<kExchangeLoad, kExchangeStore>), dim3(b.blocks), dim3(kThreads), 0, stream, b);
}

template <int L, int T>
static void launch_norm_rope_lanes(const NormRopeArgs &a, bool uniform, bool tile, uint32_t blocks,
                                   hipStream_t stream) {
    const dim3 grid(blocks), block(kRopeThreads);
    if (uniform && tile) hipLaunchKernelGGL((norm_rope_kernel<L, T, true, true>), grid, block, 0, stream, a);
    else if (uniform) hipLaunchKernelGGL((norm_rope_kernel<L, T, true, false>), grid, block, 0, stream, a);
    else if (tile) hipLaunchKernelGGL((norm_rope_kernel<L, T, false, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((norm_rope_kernel<L, T, false, false>), grid, block, 0, stream, a);
}

void launch_norm_rope_band(const NormRopeArgs &a, int dtype, uint32_t blocks, hipStream_t stream) {
    if (dtype == 2)
        hipLaunchKernelGGL(norm_rope_band_kernel<2>, dim3(blocks), dim3(kBandWaves * 64), 0, stream, a);
    else
        hipLaunchKernelGGL(norm_rope_band_kernel<1>, dim3(blocks), dim3(kBandWaves * 64), 0, stream, a);
}

void launch_norm_rope(const NormRopeArgs &a, int lanes, int dtype, bool uniform, bool tile, uint32_t blocks,
                      hipStream_t stream) {
    const bool bf = dtype == 2;
    switch (lanes) {
    case 4: bf ? launch_norm_rope_lanes<4, 2>(a, uniform, tile, blocks, stream)
               : launch_norm_rope_lanes<4, 1>(a, uniform, tile, blocks, stream); break;
    case 8: bf ? launch_norm_rope_lanes<8, 2>(a, uniform, tile, blocks, stream)
               : launch_norm_rope_lanes<8, 1>(a, uniform, tile, blocks, stream); break;
    case 16: bf ? launch_norm_rope_lanes<16, 2>(a, uniform, tile, blocks, stream)
                : launch_norm_rope_lanes<16, 1>(a, uniform, tile, blocks, stream); break;
    default: bf ? launch_norm_rope_lanes<32, 2>(a, uniform, tile, blocks, stream)
                : launch_norm_rope_lanes<32, 1>(a, uniform, tile, blocks, stream); break;
    }
}

void launch_rowmap(const RowMapArgs &a, int kind, hipStream_t stream) {
    const uint32_t blocks = (a.total + kCopyVecsPerBlock - 1) / kCopyVecsPerBlock;
    switch (kind) {
    case kPadShard:
        hipLaunchKernelGGL(rowmap_kernel<kPadShard>, dim3(blocks), dim3(kThreads), 0, stream, a);
        break;
    case kUnshardTrim:
        hipLaunchKernelGGL(rowmap_kernel<kUnshardTrim>, dim3(blocks), dim3(kThreads), 0, stream, a);
        break;
    case kSplitHalo:
        hipLaunchKernelGGL(rowmap_kernel<kSplitHalo>, dim3(blocks), dim3(kThreads), 0, stream, a);
        break;
    case kGatherStacked:
        hipLaunchKernelGGL(rowmap_kernel<kGatherStacked>, dim3(blocks), dim3(kThreads), 0, stream, a);
        break;
    default:
        hipLaunchKernelGGL(rowmap_kernel<kTrimConcat>, dim3(blocks), dim3(kThreads), 0, stream, a);
        break;
    }
}

}  // namespace uly
