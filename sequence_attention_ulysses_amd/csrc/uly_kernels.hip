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
//     already contiguous and coalesced — staging through LDS would add a
//     round trip without saving HBM traffic;
//   * no MFMA: there is no contraction on this path.
//
// Pages cited (by title and section): TeleFuser documentation,
// "Communication Architecture" ("Ulysses", "Equal-shape gather", "Spatial
// VAE Communication"); flashinfer PR #6332 ("Description", "Assumptions").

#include <hip/hip_runtime.h>

#include "uly_internal.h"

namespace uly {
namespace {

__device__ __forceinline__ uint4 load16(const void *p) {
    return *reinterpret_cast<const uint4 *>(p);
}

__device__ __forceinline__ void store16(void *p, uint4 v) {
    *reinterpret_cast<uint4 *>(p) = v;
}

// ---------------------------------------------------------------------------
// Chunk relayout (Ulysses scatter and gather, "Communication Architecture",
// "Ulysses").  Up to three operands (Q, K, V) share one launch: blocks
// [p[i].first_block, p[i+1].first_block) belong to operand i, so the three
// copies fill the machine together instead of draining one after another.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void relayout_kernel(CopyBatch b) {
    const uint32_t bid = blockIdx.x;
    int pi = 0;
    if (b.n > 1 && bid >= b.p[1].first_block) pi = 1;
    if (b.n > 2 && bid >= b.p[2].first_block) pi = 2;
    const CopyPlan &P = b.p[pi];

    const uint32_t first = (bid - P.first_block) * kCopyVecsPerBlock + threadIdx.x;
    uint4 v[kCopyUnroll];
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
            v[u] = load16(s);
        }
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const uint32_t i = first + u * kThreads;
        if (i < P.total) store16(P.dst + uint64_t(i) * 16u, v[u]);
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

template <int LANES, int DT>
__global__ __launch_bounds__(kThreads) void norm_rope_kernel(NormRopeArgs a) {
    constexpr int GROUPS = kThreads / LANES;
    const uint32_t lane = threadIdx.x % LANES;
    const uint32_t grp = threadIdx.x / LANES;
    const uint32_t half = a.D / 2;

    float w0[8], w1[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w0[i] = w1[i] = 0.f;
    if (a.op[0].w) unpack8<DT>(load16(a.op[0].w + lane * 8), w0);
    if (a.op[1].w) unpack8<DT>(load16(a.op[1].w + lane * 8), w1);

    const uint32_t row_begin = blockIdx.x * a.rows_per_block;
    const uint32_t row_end = min(row_begin + a.rows_per_block, a.rows);

    // The trip count is the same for every lane of the block; rows past
    // row_end are computed on zeros and not stored, so every lane takes
    // part in every DPP exchange.
    for (uint32_t base = row_begin; base < row_end; base += GROUPS * kRopeUnroll) {
        uint4 raw[kRopeUnroll];
        float4 cs[kRopeUnroll], sn[kRopeUnroll];
        uint16_t *dst[kRopeUnroll];
        bool second[kRopeUnroll];
#pragma unroll
        for (int k = 0; k < kRopeUnroll; ++k) {
            const uint32_t row = base + grp + k * GROUPS;
            raw[k] = make_uint4(0, 0, 0, 0);
            cs[k] = make_float4(1.f, 1.f, 1.f, 1.f);
            sn[k] = make_float4(0.f, 0.f, 0.f, 0.f);
            dst[k] = nullptr;
            second[k] = false;
            if (row < row_end) {
                uint32_t tk, hh, rb, s, r, b;
                a.rpt.divmod(row, tk, hh);
                a.sl.divmod(tk, rb, s);
                a.bdiv.divmod(rb, r, b);
                // Q or K row: select the operand's fields by value (both
                // operands stay in scalar registers).
                const bool k_op = hh >= a.H0;
                const NormRopeOperand &o0 = a.op[0], &o1 = a.op[1];
                const uint32_t h = hh - (k_op ? a.H0 : 0u);
                const uint32_t g = r * a.S_l + s;
                uint32_t qd, j;
                if (k_op) o1.hl.divmod(h, qd, j); else o0.hl.divmod(h, qd, j);
                const int64_t s_off = int64_t(r) * (k_op ? o1.s_rank : o0.s_rank) +
                                      int64_t(b) * (k_op ? o1.s_b : o0.s_b) +
                                      int64_t(s) * (k_op ? o1.s_s : o0.s_s) +
                                      int64_t(h) * (k_op ? o1.s_h : o0.s_h) + lane * 8;
                const int64_t d_off = int64_t(qd) * (k_op ? o1.d_q : o0.d_q) +
                                      int64_t(b) * (k_op ? o1.d_b : o0.d_b) +
                                      int64_t(g) * (k_op ? o1.d_g : o0.d_g) +
                                      int64_t(j) * a.D + lane * 8;
                const uint16_t *src = (k_op ? o1.src : o0.src) + s_off;
                dst[k] = (k_op ? o1.dst : o0.dst) + d_off;
                second[k] = k_op;
                raw[k] = load16(src);
                const size_t t_off = size_t(g) * half + lane * 4;
                cs[k] = *reinterpret_cast<const float4 *>(a.cos_tab + t_off);
                sn[k] = *reinterpret_cast<const float4 *>(a.sin_tab + t_off);
            }
        }
#pragma unroll
        for (int k = 0; k < kRopeUnroll; ++k) {
            float x[8];
            unpack8<DT>(raw[k], x);
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) ss = fmaf(x[i], x[i], ss);
            ss = row_sum<LANES>(ss);
            const float inv = rsqrtf(fmaf(ss, a.inv_D, a.eps));
            const float c[4] = {cs[k].x, cs[k].y, cs[k].z, cs[k].w};
            const float sv[4] = {sn[k].x, sn[k].y, sn[k].z, sn[k].w};
            uint32_t out[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const float wa = second[k] ? w1[2 * p] : w0[2 * p];
                const float wb = second[k] ? w1[2 * p + 1] : w0[2 * p + 1];
                const float n0 = x[2 * p] * inv * wa;
                const float n1 = x[2 * p + 1] * inv * wb;
                const float y0 = n0 * c[p] - n1 * sv[p];
                const float y1 = n0 * sv[p] + n1 * c[p];
                out[p] = pack2<DT>(y0, y1);
            }
            if (dst[k]) store16(dst[k], make_uint4(out[0], out[1], out[2], out[3]));
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
            if (src_row >= 0) v[u] = load16(a.src + (src_row * a.vpr.d + c) * 16);
        }
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const uint32_t i = first + u * kThreads;
        if (i < a.total) store16(a.dst + uint64_t(i) * 16u, v[u]);
    }
}

}  // namespace

void launch_relayout(const CopyBatch &b, hipStream_t stream) {
    hipLaunchKernelGGL(relayout_kernel, dim3(b.blocks), dim3(kThreads), 0, stream, b);
}

void launch_norm_rope(const NormRopeArgs &a, int lanes, int dtype, uint32_t blocks, hipStream_t stream) {
#define ULY_NR(L, T)                                                                             \
    if (lanes == L && dtype == T) {                                                              \
        hipLaunchKernelGGL((norm_rope_kernel<L, T>), dim3(blocks), dim3(kThreads), 0, stream, a); \
        return;                                                                                  \
    }
    ULY_NR(4, 1) ULY_NR(8, 1) ULY_NR(16, 1) ULY_NR(32, 1)
    ULY_NR(4, 2) ULY_NR(8, 2) ULY_NR(16, 2) ULY_NR(32, 2)
#undef ULY_NR
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
