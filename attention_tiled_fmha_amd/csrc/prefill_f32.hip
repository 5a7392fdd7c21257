// Dense prefill in fp32 end to end: the exactness test mode of the tiled
// attention (fp32 inputs, fp32 scores, fp32 softmax and accumulation).
//
// The algorithm is the tiled attention with an online softmax: K/V tiles are
// staged in LDS, each tile's scores stay on chip, the running row max m and
// row sum l are updated and the output accumulator is rescaled by
// exp(m_old - m_new) before the tile's weighted values are added (the
// FlashAttention update described in the FlashDecoding++ summary,
// wenjunhu.com/d/2311396.html, section 1, and the tiled scheme of the
// xhh.club summary, "FlashAttention and paged attention").
//
// Work split: one workgroup (256 lanes) per 16 query rows of one (b, h), 16
// lanes per query row.  A key tile holds 128 keys (D = 64) or 64 keys
// (D = 128), read with 16-byte loads, and the next tile's K and V are
// fetched into registers while the current tile is used, so a short
// sequence pays one load latency instead of one per 32 keys.  Speed is
// secondary here; precision is the aim.
#include "common.h"
#include "kernels.h"

namespace attn {

namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));

template <int D>
struct F32Cfg {
    static constexpr int BM = 16;                  // query rows per workgroup
    static constexpr int TPR = 16;                 // lanes per query row
    static constexpr int BN = D == 64 ? 128 : 64;  // keys per tile
    static constexpr int PER = BN * D / 4 / 256;   // 16-byte pieces of K (and of V) per lane
};

template <int D>
__global__ __launch_bounds__(256) void prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int Hq, int Hkv, int Tq, int Tk,
    int causal, float scale) {
    using C = F32Cfg<D>;
    constexpr int BM = C::BM, BN = C::BN, TPR = C::TPR, PER = C::PER;
    __shared__ float sQ[BM][D];
    __shared__ float sK[BN][D + 1];   // padded: the 16 lanes of a row read 16 key rows at one dim
    __shared__ __attribute__((aligned(16))) float sV[BN][D];
    __shared__ float sP[BM][BN + 1];

    const int tid = threadIdx.x;
    const int r = tid / TPR, sub = tid % TPR;
    const int n_qt = (Tq + BM - 1) / BM;
    const int q0 = (blockIdx.x % n_qt) * BM;
    const int bh = blockIdx.x / n_qt;
    const int b = bh / Hq, h = bh % Hq, kvh = h / (Hq / Hkv);
    const float* qp = q + (size_t)bh * Tq * D;
    const float* kp = k + (size_t)(b * Hkv + kvh) * Tk * D;
    const float* vp = v + (size_t)(b * Hkv + kvh) * Tk * D;

    for (int e = tid; e < BM * D / 4; e += 256) {
        const int rr = 4 * e / D, c = 4 * e % D;
        const f32x4v x = (q0 + rr < Tq) ? *(const f32x4v*)(qp + (size_t)(q0 + rr) * D + c)
                                        : f32x4v{0.f, 0.f, 0.f, 0.f};
        for (int i = 0; i < 4; i++) sQ[rr][c + i] = x[i];
    }

    const int qi = q0 + r;
    const int diag = Tk - Tq;  // causal: key j visible to query i iff j <= i + diag
    int kend = Tk;
    if (causal) kend = max(0, min(Tk, q0 + BM + diag));

    // this lane's 16-byte pieces of a tile: piece f = tid + 256 i is row
    // 4f / D, columns 4f % D .. +3; rows past Tk read as zeros
    f32x4v kr[PER], vr[PER];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int i = 0; i < PER; i++) {
            const int f = tid + 256 * i, jj = 4 * f / D, c = 4 * f % D;
            const bool in = k0 + jj < Tk;
            kr[i] = in ? *(const f32x4v*)(kp + (size_t)(k0 + jj) * D + c) : f32x4v{0.f, 0.f, 0.f, 0.f};
            vr[i] = in ? *(const f32x4v*)(vp + (size_t)(k0 + jj) * D + c) : f32x4v{0.f, 0.f, 0.f, 0.f};
        }
    };

    float m = -INFINITY, l = 0.f;
    float acc[D / TPR];
#pragma unroll
    for (int n = 0; n < D / TPR; n++) acc[n] = 0.f;

    if (kend > 0) fetch(0);
    for (int k0 = 0; k0 < kend; k0 += BN) {
        __syncthreads();  // the previous tile (and sP) is no longer read; sQ is written
#pragma unroll
        for (int i = 0; i < PER; i++) {
            const int f = tid + 256 * i, jj = 4 * f / D, c = 4 * f % D;
#pragma unroll
            for (int e = 0; e < 4; e++) sK[jj][c + e] = kr[i][e];
            *(f32x4v*)&sV[jj][c] = vr[i];
        }
        __syncthreads();
        if (k0 + BN < kend) fetch(k0 + BN);   // the next tile loads while this one is used

        float s[BN / TPR];
        float tmax = -INFINITY;
#pragma unroll
        for (int mm = 0; mm < BN / TPR; mm++) {
            const int j = sub + TPR * mm, kj = k0 + j;
            float dot = 0.f;
#pragma unroll 8
            for (int c = 0; c < D; c++) dot = fmaf(sQ[r][c], sK[j][c], dot);
            const bool visible = kj < Tk && (!causal || kj <= qi + diag);
            s[mm] = visible ? dot * scale : -INFINITY;
            tmax = fmaxf(tmax, s[mm]);
        }
#pragma unroll
        for (int off = 1; off < TPR; off <<= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, off));
        const float mnew = fmaxf(m, tmax);
        // alpha rescales what was accumulated under the old max; with no
        // visible key so far (mnew = -inf) there is nothing to rescale.
        const float alpha = (mnew == -INFINITY) ? 1.f : expf(m - mnew);
        float psum = 0.f;
#pragma unroll
        for (int mm = 0; mm < BN / TPR; mm++) {
            const float p = (s[mm] == -INFINITY) ? 0.f : expf(s[mm] - mnew);
            sP[r][sub + TPR * mm] = p;
            psum += p;
        }
#pragma unroll
        for (int off = 1; off < TPR; off <<= 1) psum += __shfl_xor(psum, off);
        l = l * alpha + psum;
        m = mnew;
        __syncthreads();
#pragma unroll
        for (int n = 0; n < D / TPR; n++) {
            const int d = sub + TPR * n;
            float a = 0.f;
#pragma unroll 8
            for (int j = 0; j < BN; j++) a = fmaf(sP[r][j], sV[j][d], a);
            acc[n] = acc[n] * alpha + a;
        }
    }

    if (qi < Tq) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        float* op = o + ((size_t)bh * Tq + qi) * D;
#pragma unroll
        for (int n = 0; n < D / TPR; n++) op[sub + TPR * n] = acc[n] * inv;
        if (lse && sub == 0) lse[(size_t)bh * Tq + qi] = l > 0.f ? m + logf(l) : -INFINITY;
    }
}

}  // namespace

hipError_t launch_prefill_f32(const float* q, const float* k, const float* v, float* o,
                              float* lse, int B, int Hq, int Hkv, int Tq, int Tk, int D,
                              bool causal, float scale, hipStream_t stream) {
    const dim3 grid(((Tq + F32Cfg<64>::BM - 1) / F32Cfg<64>::BM) * B * Hq);
    if (D == 64)
        prefill_f32_kernel<64><<<grid, 256, 0, stream>>>(q, k, v, o, lse, Hq, Hkv, Tq, Tk,
                                                         causal, scale);
    else
        prefill_f32_kernel<128><<<grid, 256, 0, stream>>>(q, k, v, o, lse, Hq, Hkv, Tq, Tk,
                                                          causal, scale);
    return hipGetLastError();
}

}  // namespace attn
