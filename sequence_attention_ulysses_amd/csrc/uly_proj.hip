// gfx950 QKV projection with the Q/K RMSNorm + interleaved RoPE + head-band
// store in its epilogue (flashinfer PR #6332, "Description": the projection,
// the per-head norm of Q and K, the rotation and the exchange in one call;
// "Assumptions": projection, then QK-norm, then RoPE, fp32 math, 16-bit
// output).
//
// The projection is the one dense contraction of the front end, so it runs
// on the matrix cores: v_mfma_f32_32x32x16_{bf16,f16}, fp32 accumulation.
// The product is computed transposed, C^T[n][t] = sum_k W[n][k] X[t][k]:
// both operands are K-contiguous rows, and the MFMA result then gives each
// lane one token and 16 head-dim values (four runs of 4) per 32x32 block.
// The RMSNorm of a (token, head) row is a sum over the lane's own registers
// plus one exchange with lane ^ 32; the rotation pairs (2j, 2j+1) sit in
// one lane's registers; one more exchange with lane ^ 32 turns the runs of 4
// into 16-byte runs for the stores.
//
// Tiling: a block of 4 waves owns one head (128 output columns, one
// component q, k or v) and 256 tokens; wave w owns tokens [64w, 64w+64), a
// 128 x 64 tile of 4 x 2 MFMA blocks (128 fp32 accumulators per lane).  K
// advances 32 at a time through a two-stage LDS ring; the global loads of
// stage k+2 are in flight while stage k is multiplied.  LDS rows are 64
// bytes (four 16-byte chunks) with the chunk index XOR-swizzled by row, so
// the 16-byte fragment reads of 32 consecutive rows do not collide on banks.

#include <hip/hip_runtime.h>

#include "uly.h"
#include "uly_internal.h"

namespace uly {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) u32x4_t global_u32x4_t;

constexpr int kWaves = kProjThreads / 64;
constexpr int kChunks = kProjTileK / 8;                  // 16-byte chunks per LDS row
constexpr int kRowsA = kProjD;                           // weight rows per block
constexpr int kRowsB = kProjTileT;                       // token rows per block
constexpr int kLoadsA = kRowsA * kChunks / kProjThreads; // 16-byte loads per thread per stage
constexpr int kLoadsB = kRowsB * kChunks / kProjThreads;
static_assert(kChunks == 4, "the LDS swizzle assumes 64-byte rows");
static_assert(kRowsA * kChunks % kProjThreads == 0 && kRowsB * kChunks % kProjThreads == 0, "tile split");
static_assert(kProjTileT == kWaves * 64, "each wave owns 64 tokens");

__device__ __forceinline__ uint4 ldg16(const uint16_t *p) {
    const u32x4_t v = *(const global_u32x4_t *)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void stg16(uint16_t *p, uint4 v) {
    const u32x4_t w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, (global_u32x4_t *)p);
}

// LDS slot of 16-byte chunk c of row `row`.
__device__ __forceinline__ int swz(int row, int c) { return row * kChunks + (c ^ ((row >> 1) & 3)); }

template <int DT>
__device__ __forceinline__ f32x16_t mfma(uint4 a, uint4 b, f32x16_t c) {
    if constexpr (DT == 2)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
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

template <int DT>
__global__ __launch_bounds__(kProjThreads) void proj_norm_rope_kernel(ProjArgs a) {
    __shared__ uint4 sA[2][kRowsA * kChunks];
    __shared__ uint4 sB[2][kRowsB * kChunks];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    uint32_t tile, hd;
    a.nh.divmod(blockIdx.x, tile, hd);                  // heads fastest: a token tile stays hot in L2
    const uint32_t m0 = tile * kProjTileT;
    const uint16_t *wrow = a.w + size_t(hd) * kProjD * a.K;

    // Global -> register staging of one K stage.  Rows past M read row M-1.
    uint4 ra[kLoadsA], rb[kLoadsB];
    auto gload = [&](uint32_t kt) {
        const uint32_t k0 = kt * kProjTileK;
#pragma unroll
        for (int u = 0; u < kLoadsA; ++u) {
            const int i = tid + u * kProjThreads;
            ra[u] = ldg16(wrow + size_t(i / kChunks) * a.K + k0 + (i % kChunks) * 8);
        }
#pragma unroll
        for (int u = 0; u < kLoadsB; ++u) {
            const int i = tid + u * kProjThreads;
            const uint32_t m = min(m0 + uint32_t(i / kChunks), a.M - 1);
            rb[u] = ldg16(a.x + size_t(m) * a.K + k0 + (i % kChunks) * 8);
        }
    };
    auto sstore = [&](int st) {
#pragma unroll
        for (int u = 0; u < kLoadsA; ++u) {
            const int i = tid + u * kProjThreads;
            sA[st][swz(i / kChunks, i % kChunks)] = ra[u];
        }
#pragma unroll
        for (int u = 0; u < kLoadsB; ++u) {
            const int i = tid + u * kProjThreads;
            sB[st][swz(i / kChunks, i % kChunks)] = rb[u];
        }
    };

    f32x16_t acc[4][2];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[nb][tb][i] = 0.f;

    const uint32_t KT = a.K / kProjTileK;
    gload(0);
    sstore(0);
    if (KT > 1) gload(1);
    __syncthreads();
    const int fr = lane & 31;          // fragment row (A) / column (B) of this lane
    const int fk = lane >> 5;          // which 8-wide half of a 16-wide K step
    for (uint32_t kt = 0; kt < KT; ++kt) {
        const int st = kt & 1;
        if (kt + 1 < KT) sstore(st ^ 1);   // stage kt+1, read back after the barrier below
        if (kt + 2 < KT) gload(kt + 2);    // in flight during this stage's products
#pragma unroll
        for (int ks = 0; ks < kProjTileK / 16; ++ks) {
            const int c = ks * 2 + fk;
            uint4 fa[4], fb[2];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) fa[nb] = sA[st][swz(nb * 32 + fr, c)];
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) fb[tb] = sB[st][swz(wv * 64 + tb * 32 + fr, c)];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) acc[nb][tb] = mfma<DT>(fa[nb], fb[tb], acc[nb][tb]);
        }
        __syncthreads();
    }

    // ---- epilogue -----------------------------------------------------------
    // acc[nb][tb][i] is column n = 32nb + 8(i/4) + 4*half + i%4 (the head-dim
    // index d) of token 64wv + 32tb + lane%32.
    const uint32_t half = lane >> 5;
    const int comp = hd < a.Hq ? 0 : (hd < a.Hq + a.Hkv ? 1 : 2);
    const uint32_t hc = hd - (comp == 0 ? 0u : (comp == 1 ? a.Hq : a.Hq + a.Hkv));
    uint32_t qd, jd;
    a.hl[comp].divmod(hc, qd, jd);
    const uint16_t *wn = comp < 2 ? a.wn[comp] : nullptr;
    uint16_t *dbase = a.dst[comp] + int64_t(qd) * a.d_q[comp] + int64_t(jd) * kProjD;
    const int64_t d_b = a.d_b[comp], d_g = a.d_g[comp];

#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const uint32_t tok = m0 + wv * 64 + tb * 32 + (lane & 31);
        const bool live = tok < a.M;
        uint32_t rb_, s, r, b;
        a.sl.divmod(live ? tok : a.M - 1, rb_, s);
        a.bdiv.divmod(rb_, r, b);
        const uint32_t g = r * a.S_l + s;
        float inv = 1.f;
        if (comp < 2) {
            float ss = 0.f;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int i = 0; i < 16; ++i) ss = fmaf(acc[nb][tb][i], acc[nb][tb][i], ss);
            ss += __shfl_xor(ss, 32, 64);
            // eps > 0 keeps the argument normal: the bare reciprocal square root suffices
            inv = __builtin_amdgcn_rsqf(fmaf(ss, a.inv_D, a.eps));
        }
        uint16_t *drow = dbase + int64_t(b) * d_b + int64_t(g) * d_g;
        const float *crow = a.cos_tab + size_t(g) * (kProjD / 2);
        const float *srow = a.sin_tab + size_t(g) * (kProjD / 2);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            uint32_t pk[8];   // pk[2*grp + p]: the pair (d0 + 2p, d0 + 2p + 1) of register group grp
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                const int d0 = nb * 32 + grp * 8 + int(half) * 4;
                if (comp < 2) {
                    const float2 cc = *(const float2 *)(crow + d0 / 2);
                    const float2 sn = *(const float2 *)(srow + d0 / 2);
                    const uint2 wr = *(const uint2 *)(wn + d0);
                    const float wf[4] = {widen1<DT>(wr.x & 0xFFFFu), widen1<DT>(wr.x >> 16),
                                         widen1<DT>(wr.y & 0xFFFFu), widen1<DT>(wr.y >> 16)};
                    const float cv[2] = {cc.x, cc.y}, sv[2] = {sn.x, sn.y};
#pragma unroll
                    for (int p = 0; p < 2; ++p) {
                        const int i0 = grp * 4 + p * 2;
                        const float n0 = acc[nb][tb][i0] * inv * wf[2 * p];
                        const float n1 = acc[nb][tb][i0 + 1] * inv * wf[2 * p + 1];
                        pk[grp * 2 + p] = pack2<DT>(n0 * cv[p] - n1 * sv[p], n0 * sv[p] + n1 * cv[p]);
                    }
                } else {
#pragma unroll
                    for (int p = 0; p < 2; ++p)
                        pk[grp * 2 + p] = pack2<DT>(acc[nb][tb][grp * 4 + p * 2], acc[nb][tb][grp * 4 + p * 2 + 1]);
                }
            }
            // Lane half 0 holds d runs {0-3, 8-11, 16-19, 24-27} (+32nb), half 1 the
            // runs 4 higher; one exchange gives half 0 d 0-7 and 16-23, half 1 d 8-15
            // and 24-31, each a 16-byte run.
            uint32_t snd[4], rcv[4];
            snd[0] = half ? pk[0] : pk[2];
            snd[1] = half ? pk[1] : pk[3];
            snd[2] = half ? pk[4] : pk[6];
            snd[3] = half ? pk[5] : pk[7];
#pragma unroll
            for (int i = 0; i < 4; ++i) rcv[i] = __shfl_xor(snd[i], 32, 64);
            const uint4 lo = half ? make_uint4(rcv[0], rcv[1], pk[2], pk[3]) : make_uint4(pk[0], pk[1], rcv[0], rcv[1]);
            const uint4 hi = half ? make_uint4(rcv[2], rcv[3], pk[6], pk[7]) : make_uint4(pk[4], pk[5], rcv[2], rcv[3]);
            if (live) {
                stg16(drow + nb * 32 + half * 8, lo);
                stg16(drow + nb * 32 + 16 + half * 8, hi);
            }
        }
    }
}

}  // namespace

void launch_proj(const ProjArgs &a, int dtype, uint32_t blocks, hipStream_t stream) {
    if (dtype == ULY_BF16)
        hipLaunchKernelGGL(proj_norm_rope_kernel<2>, dim3(blocks), dim3(kProjThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(proj_norm_rope_kernel<1>, dim3(blocks), dim3(kProjThreads), 0, stream, a);
}

}  // namespace uly
