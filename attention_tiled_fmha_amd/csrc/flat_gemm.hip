// Flat GEMM of the decode phase on gfx950 MFMA: C = A W^T.
//
// In decode every projection (K/Q/V, O, the two FFN layers) multiplies the
// few tokens of a step, A [m][k] with m = the batch size, by a weight
// W [n][k]; the product is "flat" (m << n, k) and its time is the time to
// read W once.  The FlashDecoding++ summary (wenjunhu.com/d/2311396.html,
// sections 1 and 4) pads such an m only to the matrix unit's smallest tile
// instead of 64 and hides the memory latency with double buffering; section 5
// picks the kernel's parameters from m, n and k.
//
// gfx950 mapping
// --------------
// C^T = W A^T on v_mfma_f32_16x16x32_bf16: 16 rows of W are the A operand,
// up to 16 tokens of A are the (zero-padded) B operand, so m is padded to 16
// (MT = ceil(m / 16) <= 4 token tiles share every W fragment).  Per 32-wide k
// step lane l loads 16 bytes of W row l % 16 (k = 32 step + 8 (l / 16) .. +7)
// and, per token tile t, 16 bytes of token 16 t + l % 16 at the same k, which
// is the operands' register order, so nothing is shuffled.  Four lanes read
// 64 contiguous bytes of a row; the next step reads the next 64.
//
// A workgroup (4 or 8 wavefronts) owns RB = 1, 2 or 4 row blocks of 16 rows
// of W, all of which use the same A fragments; its k range (all of k, or one
// of `splits` slices) is cut into contiguous per-wavefront ranges.  Each
// wavefront streams its range in batches of U steps with the next batch's
// loads in flight while the current batch's MFMAs run: double buffering in
// registers, since every byte of W is used once and staging it through LDS
// would only add traffic.  The wavefronts' partial products are summed in
// fixed order through LDS.  With
// splits > 1 each slice writes fp32 partials to the workspace and
// flat_gemm_reduce_kernel adds them in slice order.
//
// Loads are raw buffer loads.  W's descriptor covers only the workgroup's
// valid rows and A's only the m tokens, so padded rows and tokens read zeros
// with no branch; a step past the wavefront's range or past k gets an offset
// beyond every descriptor and reads zeros too (adding exact zeros), so the
// loop has no conditionals.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace attn {

namespace {

constexpr int kRsrcWord3 = 0x00020000;     // raw 32-bit data, no swizzle
constexpr int kOutOfRange = 0x7fffff00;    // an offset past every descriptor's size

template <int MT, int RB, int U>
struct Batch {
    u32x4 w[U][RB];
    u32x4 a[U][MT];
};

// RB 16-row blocks of W per workgroup (the same A fragments serve all of
// them), MT token tiles, U k steps per register batch, NW wavefronts.
template <int MT, int RB, int U, int NW, bool OUT_F32>
__global__ __launch_bounds__(NW * 64) void flat_gemm_kernel(
    const uint16_t* __restrict__ a, const uint16_t* __restrict__ w, void* __restrict__ c,
    float* __restrict__ ws, int m, int n, int k, int splits, int steps_per_split) {
    constexpr int kFgWaves = NW;
    constexpr int kFgThreads = NW * 64;
    __shared__ __attribute__((aligned(16))) f32x4 red[kFgWaves][MT][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, g = lane >> 4;

    const int rb = blockIdx.x / splits, split = blockIdx.x % splits;
    const int n0 = rb * 16 * RB;
    const int rows = min(16 * RB, n - n0);
    const int nsteps = (k + 31) / 32;
    const int s0 = split * steps_per_split;
    const int s1 = min(nsteps, s0 + steps_per_split);
    const int per_wave = (s1 - s0 + kFgWaves - 1) / kFgWaves;
    const int ws0 = s0 + wave * per_wave;
    const int ws1 = min(s1, ws0 + per_wave);

    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(w + (size_t)n0 * k), (short)0, rows * k * 2, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a, (short)0, m * k * 2, kRsrcWord3);

    // this lane's fragments of the U steps from st0
    auto load = [&](Batch<MT, RB, U>& bt, int st0) {
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int kk = 32 * (st0 + u) + 8 * g;
            const bool ok = (st0 + u < ws1) && (kk < k);
#pragma unroll
            for (int r = 0; r < RB; r++) {
                const int ow = ok ? ((16 * r + col) * k + kk) * 2 : kOutOfRange;
                bt.w[u][r] = __builtin_amdgcn_raw_buffer_load_b128(rw, ow, 0, 0);
            }
#pragma unroll
            for (int t = 0; t < MT; t++) {
                const int oa = ok ? ((16 * t + col) * k + kk) * 2 : kOutOfRange;
                bt.a[u][t] = __builtin_amdgcn_raw_buffer_load_b128(ra, oa, 0, 0);
            }
        }
    };

    f32x4 acc[RB][MT];
#pragma unroll
    for (int r = 0; r < RB; r++)
#pragma unroll
        for (int t = 0; t < MT; t++) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](const Batch<MT, RB, U>& bt) {
#pragma unroll
        for (int u = 0; u < U; u++)
#pragma unroll
            for (int r = 0; r < RB; r++)
#pragma unroll
                for (int t = 0; t < MT; t++)
                    acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, bt.w[u][r]),
                        __builtin_bit_cast(bf16x8, bt.a[u][t]), acc[r][t], 0, 0, 0);
    };

    // batches of U steps; the batch after the last one loads out-of-range
    // offsets only (zeros, no memory traffic)
    const int nb = ws1 > ws0 ? (ws1 - ws0 + U - 1) / U : 0;
    Batch<MT, RB, U> b0, b1;
    if (nb > 0) load(b0, ws0);
    int i = 0;
    for (; i + 1 < nb; i += 2) {
        load(b1, ws0 + (i + 1) * U);
        compute(b0);
        load(b0, ws0 + (i + 2) * U);
        compute(b1);
    }
    if (i < nb) compute(b0);

    // per row block: sum the wavefronts' partial products in wave order
#pragma unroll
    for (int r = 0; r < RB; r++) {
        if (r > 0) __syncthreads();   // the previous block's sums have been read
#pragma unroll
        for (int t = 0; t < MT; t++) red[wave][t][lane] = acc[r][t];
        __syncthreads();
        for (int e = tid; e < MT * 64 * 4; e += kFgThreads) {
            const int q = e & 3, l = (e >> 2) & 63, t = e >> 8;
            float s = 0.f;
#pragma unroll
            for (int v = 0; v < kFgWaves; v++) s += red[v][t][l][q];
            const int token = 16 * t + (l & 15);
            const int nrow = n0 + 16 * r + 4 * (l >> 4) + q;
            if (token < m && nrow < n) {
                if (splits > 1)
                    ws[((size_t)split * m + token) * n + nrow] = s;
                else if (OUT_F32)
                    ((float*)c)[(size_t)token * n + nrow] = s;
                else
                    ((uint16_t*)c)[(size_t)token * n + nrow] = f32_to_bf16(s);
            }
        }
    }
}

// C = the sum of the `splits` fp32 partials, added in slice order.
template <bool OUT_F32>
__global__ __launch_bounds__(256) void flat_gemm_reduce_kernel(const float* __restrict__ ws,
                                                               void* __restrict__ c, long mn,
                                                               int splits) {
    for (long e = blockIdx.x * 256L + threadIdx.x; e < mn; e += (long)gridDim.x * 256) {
        float s = 0.f;
        for (int p = 0; p < splits; p++) s += ws[(size_t)p * mn + e];
        if (OUT_F32)
            ((float*)c)[e] = s;
        else
            ((uint16_t*)c)[e] = f32_to_bf16(s);
    }
}

// Steps per register batch: the loads of two batches stay within ~130 VGPRs.
template <int MT, int RB> struct BatchSteps {
    static constexpr int U = RB == 1 ? (MT == 1 ? 8 : MT == 2 ? 4 : 2)
                           : RB == 2 ? (MT == 1 ? 4 : 2)
                                     : (MT <= 2 ? 2 : 1);
};

template <int MT, int RB, int NW, bool OUT_F32>
hipError_t go_nw(const FlatGemmArgs& p, hipStream_t stream) {
    constexpr int U = BatchSteps<MT, RB>::U;
    const int rblocks = (p.n + 16 * RB - 1) / (16 * RB);
    flat_gemm_kernel<MT, RB, U, NW, OUT_F32><<<dim3(rblocks * p.splits), NW * 64, 0, stream>>>(
        (const uint16_t*)p.a, (const uint16_t*)p.w, p.c, p.ws, p.m, p.n, p.k, p.splits,
        p.steps_per_split);
    if (p.splits > 1) {
        const long mn = (long)p.m * p.n;
        const int blocks = (int)std::min<long>((mn + 255) / 256, 4096);
        flat_gemm_reduce_kernel<OUT_F32><<<blocks, 256, 0, stream>>>(p.ws, p.c, mn, p.splits);
    }
    return hipGetLastError();
}

template <int MT, int RB, bool OUT_F32>
hipError_t go(const FlatGemmArgs& p, hipStream_t stream) {
    if (p.waves == 8) return go_nw<MT, RB, 8, OUT_F32>(p, stream);
    return go_nw<MT, RB, 4, OUT_F32>(p, stream);
}

template <int RB, bool OUT_F32>
hipError_t go_mt(const FlatGemmArgs& p, hipStream_t stream) {
    switch ((p.m + 15) / 16) {
        case 1: return go<1, RB, OUT_F32>(p, stream);
        case 2: return go<2, RB, OUT_F32>(p, stream);
        case 3: return go<3, RB, OUT_F32>(p, stream);
        default: return go<4, RB, OUT_F32>(p, stream);
    }
}

template <int RB>
int batch_steps(int m) {
    switch ((m + 15) / 16) {
        case 1: return BatchSteps<1, RB>::U;
        case 2: return BatchSteps<2, RB>::U;
        case 3: return BatchSteps<3, RB>::U;
        default: return BatchSteps<4, RB>::U;
    }
}

}  // namespace

int flat_gemm_batch_steps(int m, int row_blocks) {
    return row_blocks == 4 ? batch_steps<4>(m) : row_blocks == 2 ? batch_steps<2>(m) : batch_steps<1>(m);
}

hipError_t launch_flat_gemm(const FlatGemmArgs& p, hipStream_t stream) {
    if (p.row_blocks == 4) return p.out_f32 ? go_mt<4, true>(p, stream) : go_mt<4, false>(p, stream);
    if (p.row_blocks == 2) return p.out_f32 ? go_mt<2, true>(p, stream) : go_mt<2, false>(p, stream);
    return p.out_f32 ? go_mt<1, true>(p, stream) : go_mt<1, false>(p, stream);
}

}  // namespace attn
