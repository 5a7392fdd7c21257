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

#define LDS_AS __attribute__((address_space(3)))

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

// ---------------------------------------------------------------------------
// LDS-tiled variant for m > 16 (two to four token tiles).
//
// With 64 rows of W per workgroup the register-streaming kernel above reads
// as many bytes of A (from L2) as of W, and every W load instruction touches
// 16 rows x 64 bytes; at m = 64 both keep it near 2.5 TB/s.  Here a
// workgroup owns TR = 64, 128 or 256 rows of W (RBW 16-row blocks per
// wavefront) and walks its k range in chunks of 64: the chunk's W tile
// [TR][64] and A tile [64][64] go from HBM straight into LDS (buffer loads
// with the LDS destination; each load instruction fills 1 KiB of LDS from
// 16-byte granules of consecutive rows), double-buffered, and all four
// wavefronts take their MFMA operands from the one A tile.  A is then read
// once per TR rows, W in whole 128-byte row pieces.
//
// LDS rows are 128 bytes (8 granules of 16 bytes); granule p of row r sits
// at position p ^ ((r / 2) mod 8), so the 16 rows one operand read spans hit
// 16 distinct 16-byte bank groups.  The loads fetch the global granule that
// belongs at each LDS position.  Granules past k (k is a multiple of 8, so a
// granule is all in or all out), rows past n and tokens past m get an offset
// beyond their descriptor and land as zeros.
//
// Per chunk a wavefront runs 2 k steps x RBW row blocks x MT token tiles of
// v_mfma_f32_16x16x32_bf16 (A operand W from LDS, B operand A from LDS).
// Each wavefront owns its rows outright, so it writes its results with no
// cross-wavefront reduction: C (or, with k slices, fp32 partials that
// flat_gemm_reduce_kernel adds in slice order).
constexpr int kKC = 64;                  // k per chunk (two 32-wide MFMA steps)
constexpr int kRowBytes = 2 * kKC;       // bytes of one row of a chunk tile

__device__ __forceinline__ int fg_swz(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ void fg_lds_load16(__amdgpu_buffer_rsrc_t r, unsigned char LDS_AS* dst,
                                              int off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void LDS_AS*)dst, 16, off, 0, 0, 0);
}

template <int MT, int RBW, bool OUT_F32>
__global__ __launch_bounds__(256) void flat_gemm_lds_kernel(
    const uint16_t* __restrict__ a, const uint16_t* __restrict__ w, void* __restrict__ c,
    float* __restrict__ ws, int m, int n, int k, int splits, int chunks_per_split) {
    constexpr int TR = 64 * RBW;                  // rows of W per workgroup
    constexpr int WT = TR * kRowBytes;            // bytes of a W chunk tile
    constexpr int AT = 64 * kRowBytes;            // bytes of an A chunk tile (64 token rows)
    constexpr int WL = WT / 4096;                 // W loads per thread per chunk
    constexpr int AL = AT / 4096;                 // A loads per thread per chunk
    // two stages, each its own LDS object, so that reads of one stage wait
    // only for the loads into that stage
    __shared__ __attribute__((aligned(1024))) unsigned char w_st0[WT];
    __shared__ __attribute__((aligned(1024))) unsigned char w_st1[WT];
    __shared__ __attribute__((aligned(1024))) unsigned char a_st0[AT];
    __shared__ __attribute__((aligned(1024))) unsigned char a_st1[AT];
    unsigned char LDS_AS* const sW[2] = {(unsigned char LDS_AS*)w_st0, (unsigned char LDS_AS*)w_st1};
    unsigned char LDS_AS* const sA[2] = {(unsigned char LDS_AS*)a_st0, (unsigned char LDS_AS*)a_st1};

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, g = lane >> 4;

    const int tile = blockIdx.x / splits, split = blockIdx.x % splits;
    const int n0 = tile * TR;
    const int rows = min(TR, n - n0);
    const int nchunks = (k + kKC - 1) / kKC;
    const int c0 = split * chunks_per_split;
    const int c1 = min(nchunks, c0 + chunks_per_split);

    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(w + (size_t)n0 * k), (short)0, rows * k * 2, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a, (short)0, m * k * 2, kRsrcWord3);

    // this thread's granules: g = tid + 256 j sits at LDS byte 16 g (row g / 8,
    // position g % 8) and holds global granule (g % 8) ^ swz(row) of the row
    int w_row[WL], w_gp[WL], a_row[AL], a_gp[AL];
#pragma unroll
    for (int j = 0; j < WL; j++) {
        const int gi = tid + 256 * j;
        w_row[j] = gi >> 3;
        w_gp[j] = (gi & 7) ^ fg_swz(gi >> 3);
    }
#pragma unroll
    for (int j = 0; j < AL; j++) {
        const int gi = tid + 256 * j;
        a_row[j] = gi >> 3;
        a_gp[j] = (gi & 7) ^ fg_swz(gi >> 3);
    }
    // loads of chunk ch into stage st (every thread issues WL + AL loads)
    auto issue = [&](int ch, int st) {
#pragma unroll
        for (int j = 0; j < WL; j++) {
            const int kk = ch * kKC + 8 * w_gp[j];
            const int off = kk < k ? (w_row[j] * k + kk) * 2 : kOutOfRange;
            fg_lds_load16(rw, sW[st] + 1024 * (wave + 4 * j), off);
        }
#pragma unroll
        for (int j = 0; j < AL; j++) {
            const int kk = ch * kKC + 8 * a_gp[j];
            const int off = kk < k ? (a_row[j] * k + kk) * 2 : kOutOfRange;
            fg_lds_load16(ra, sA[st] + 1024 * (wave + 4 * j), off);
        }
    };

    f32x4 acc[RBW][MT];
#pragma unroll
    for (int r = 0; r < RBW; r++)
#pragma unroll
        for (int t = 0; t < MT; t++) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // operand reads: row block r of this wavefront (rows 16 (RBW wave + r) +
    // col) and token tile t (tokens 16 t + col), k granule 4 s + g
    auto compute = [&](int st) {
        const unsigned char LDS_AS* sw = sW[st];
        const unsigned char LDS_AS* sa = sA[st];
#pragma unroll
        for (int s2 = 0; s2 < 2; s2++) {
            bf16x8 wf[RBW], af[MT];
#pragma unroll
            for (int r = 0; r < RBW; r++) {
                const int row = 16 * (RBW * wave + r) + col;
                wf[r] = *(const bf16x8 LDS_AS*)(sw + row * kRowBytes + 16 * ((4 * s2 + g) ^ fg_swz(row)));
            }
#pragma unroll
            for (int t = 0; t < MT; t++) {
                const int tok = 16 * t + col;
                af[t] = *(const bf16x8 LDS_AS*)(sa + tok * kRowBytes + 16 * ((4 * s2 + g) ^ fg_swz(tok)));
            }
#pragma unroll
            for (int r = 0; r < RBW; r++)
#pragma unroll
                for (int t = 0; t < MT; t++)
                    acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[r], af[t], acc[r][t], 0, 0, 0);
        }
    };
    // this thread's loads of the chunk issued last may stay in flight; the
    // earlier chunk's have landed, and after the barrier every thread's have
    auto wait_prev = [&]() {
        if constexpr (WL + AL == 10) asm volatile("s_waitcnt vmcnt(10)\n\ts_barrier" ::: "memory");
        else if constexpr (WL + AL == 6) asm volatile("s_waitcnt vmcnt(6)\n\ts_barrier" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
    };
    auto lds_barrier = [&]() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

    if (c1 > c0) {
        issue(c0, 0);
        int ch = c0;
        // chunk ch in stage (ch - c0) % 2: its loads were issued one chunk
        // earlier; the next chunk's loads go out before its MFMAs
        for (; ch + 1 < c1; ch += 2) {
            issue(ch + 1, 1);
            wait_prev();
            compute(0);
            lds_barrier();                 // stage 0 is rewritten next
            if (ch + 2 < c1) issue(ch + 2, 0);
            if (ch + 2 < c1) wait_prev();
            else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
            compute(1);
            lds_barrier();                 // stage 1 is rewritten next
        }
        if (ch < c1) {                     // an odd count: the last chunk, in stage 0
            asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
            compute(0);
        }
    }

    // C^T block (row block r, token tile t): lane l holds rows 4 g + q of the
    // block for token 16 t + col, i.e. 4 consecutive columns of C, stored as
    // one vector when n and the output pointer allow it
    const bool vec = (n & 3) == 0 &&
                     ((splits > 1) || ((size_t)c & (OUT_F32 ? 15 : 7)) == 0);
#pragma unroll
    for (int r = 0; r < RBW; r++) {
        const int nrow0 = n0 + 16 * (RBW * wave + r) + 4 * g;
#pragma unroll
        for (int t = 0; t < MT; t++) {
            const int token = 16 * t + col;
            if (token >= m) continue;
            const f32x4 v = acc[r][t];
            if (splits > 1) {
                float* dst = ws + ((size_t)split * m + token) * n + nrow0;
                if (vec && nrow0 + 3 < n) *(f32x4*)dst = v;
                else
                    for (int q = 0; q < 4; q++)
                        if (nrow0 + q < n) dst[q] = v[q];
            } else if (OUT_F32) {
                float* dst = (float*)c + (size_t)token * n + nrow0;
                if (vec && nrow0 + 3 < n) *(f32x4*)dst = v;
                else
                    for (int q = 0; q < 4; q++)
                        if (nrow0 + q < n) dst[q] = v[q];
            } else {
                uint16_t* dst = (uint16_t*)c + (size_t)token * n + nrow0;
                if (vec && nrow0 + 3 < n)
                    *(u32x2*)dst = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                else
                    for (int q = 0; q < 4; q++)
                        if (nrow0 + q < n) dst[q] = f32_to_bf16(v[q]);
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

template <int MT, int RBW, bool OUT_F32>
hipError_t go_lds(const FlatGemmArgs& p, hipStream_t stream) {
    const int tiles = (p.n + 64 * RBW - 1) / (64 * RBW);
    flat_gemm_lds_kernel<MT, RBW, OUT_F32><<<dim3(tiles * p.splits), 256, 0, stream>>>(
        (const uint16_t*)p.a, (const uint16_t*)p.w, p.c, p.ws, p.m, p.n, p.k, p.splits,
        p.chunks_per_split);
    if (p.splits > 1) {
        const long mn = (long)p.m * p.n;
        const int blocks = (int)std::min<long>((mn + 255) / 256, 4096);
        flat_gemm_reduce_kernel<OUT_F32><<<blocks, 256, 0, stream>>>(p.ws, p.c, mn, p.splits);
    }
    return hipGetLastError();
}

template <int RBW, bool OUT_F32>
hipError_t go_lds_mt(const FlatGemmArgs& p, hipStream_t stream) {
    switch ((p.m + 15) / 16) {
        case 1: return go_lds<1, RBW, OUT_F32>(p, stream);
        case 2: return go_lds<2, RBW, OUT_F32>(p, stream);
        case 3: return go_lds<3, RBW, OUT_F32>(p, stream);
        default: return go_lds<4, RBW, OUT_F32>(p, stream);
    }
}

template <bool OUT_F32>
hipError_t launch_lds(const FlatGemmArgs& p, hipStream_t stream) {
    if (p.lds_rows == 256) return go_lds_mt<4, OUT_F32>(p, stream);
    if (p.lds_rows == 128) return go_lds_mt<2, OUT_F32>(p, stream);
    return go_lds_mt<1, OUT_F32>(p, stream);
}

hipError_t launch_flat_gemm(const FlatGemmArgs& p, hipStream_t stream) {
    if (p.lds_rows > 0) return p.out_f32 ? launch_lds<true>(p, stream) : launch_lds<false>(p, stream);
    if (p.row_blocks == 4) return p.out_f32 ? go_mt<4, true>(p, stream) : go_mt<4, false>(p, stream);
    if (p.row_blocks == 2) return p.out_f32 ? go_mt<2, true>(p, stream) : go_mt<2, false>(p, stream);
    return p.out_f32 ? go_mt<1, true>(p, stream) : go_mt<1, false>(p, stream);
}

}  // namespace attn
