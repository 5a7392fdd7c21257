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
// Work split: one workgroup (256 lanes) per 32 query rows of one (b, h);
// 8 lanes per query row.  Speed is not the aim of this kernel; precision is.
#include "common.h"
#include "kernels.h"

namespace attn {

namespace {

constexpr int kBM = 32;   // query rows per workgroup
constexpr int kBN = 32;   // keys per tile
constexpr int kTPR = 8;   // lanes per query row

template <int D>
__global__ __launch_bounds__(256) void prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int Hq, int Hkv, int Tq, int Tk,
    int causal, float scale) {
    __shared__ float sQ[kBM][D];
    __shared__ float sK[kBN][D + 1];
    __shared__ float sV[kBN][D];
    __shared__ float sP[kBM][kBN + 1];

    const int tid = threadIdx.x;
    const int r = tid / kTPR, sub = tid % kTPR;
    const int n_qt = (Tq + kBM - 1) / kBM;
    const int q0 = (blockIdx.x % n_qt) * kBM;
    const int bh = blockIdx.x / n_qt;
    const int b = bh / Hq, h = bh % Hq, kvh = h / (Hq / Hkv);
    const float* qp = q + (size_t)bh * Tq * D;
    const float* kp = k + (size_t)(b * Hkv + kvh) * Tk * D;
    const float* vp = v + (size_t)(b * Hkv + kvh) * Tk * D;

    for (int e = tid; e < kBM * D; e += 256) {
        const int rr = e / D, c = e % D;
        sQ[rr][c] = (q0 + rr < Tq) ? qp[(size_t)(q0 + rr) * D + c] : 0.f;
    }

    const int qi = q0 + r;
    const int diag = Tk - Tq;  // causal: key j visible to query i iff j <= i + diag
    int kend = Tk;
    if (causal) kend = max(0, min(Tk, q0 + kBM + diag));

    float m = -INFINITY, l = 0.f;
    float acc[D / kTPR];
#pragma unroll
    for (int n = 0; n < D / kTPR; n++) acc[n] = 0.f;

    for (int k0 = 0; k0 < kend; k0 += kBN) {
        __syncthreads();  // the previous tile is no longer read
        for (int e = tid; e < kBN * D; e += 256) {
            const int jj = e / D, c = e % D;
            const bool in = k0 + jj < Tk;
            sK[jj][c] = in ? kp[(size_t)(k0 + jj) * D + c] : 0.f;
            sV[jj][c] = in ? vp[(size_t)(k0 + jj) * D + c] : 0.f;
        }
        __syncthreads();

        float s[kBN / kTPR];
        float tmax = -INFINITY;
#pragma unroll
        for (int mm = 0; mm < kBN / kTPR; mm++) {
            const int j = sub + kTPR * mm, kj = k0 + j;
            float dot = 0.f;
#pragma unroll 8
            for (int c = 0; c < D; c++) dot = fmaf(sQ[r][c], sK[j][c], dot);
            const bool visible = kj < Tk && (!causal || kj <= qi + diag);
            s[mm] = visible ? dot * scale : -INFINITY;
            tmax = fmaxf(tmax, s[mm]);
        }
#pragma unroll
        for (int off = 1; off < kTPR; off <<= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, off));
        const float mnew = fmaxf(m, tmax);
        // alpha rescales what was accumulated under the old max; with no
        // visible key so far (mnew = -inf) there is nothing to rescale.
        const float alpha = (mnew == -INFINITY) ? 1.f : expf(m - mnew);
        float psum = 0.f;
#pragma unroll
        for (int mm = 0; mm < kBN / kTPR; mm++) {
            const float p = (s[mm] == -INFINITY) ? 0.f : expf(s[mm] - mnew);
            sP[r][sub + kTPR * mm] = p;
            psum += p;
        }
#pragma unroll
        for (int off = 1; off < kTPR; off <<= 1) psum += __shfl_xor(psum, off);
        l = l * alpha + psum;
        m = mnew;
        __syncthreads();
#pragma unroll
        for (int n = 0; n < D / kTPR; n++) {
            const int d = sub + kTPR * n;
            float a = 0.f;
#pragma unroll 8
            for (int j = 0; j < kBN; j++) a = fmaf(sP[r][j], sV[j][d], a);
            acc[n] = acc[n] * alpha + a;
        }
    }

    if (qi < Tq) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        float* op = o + ((size_t)bh * Tq + qi) * D;
#pragma unroll
        for (int n = 0; n < D / kTPR; n++) op[sub + kTPR * n] = acc[n] * inv;
        if (lse && sub == 0) lse[(size_t)bh * Tq + qi] = l > 0.f ? m + logf(l) : -INFINITY;
    }
}

}  // namespace

hipError_t launch_prefill_f32(const float* q, const float* k, const float* v, float* o,
                              float* lse, int B, int Hq, int Hkv, int Tq, int Tk, int D,
                              bool causal, float scale, hipStream_t stream) {
    const dim3 grid(((Tq + kBM - 1) / kBM) * B * Hq);
    if (D == 64)
        prefill_f32_kernel<64><<<grid, 256, 0, stream>>>(q, k, v, o, lse, Hq, Hkv, Tq, Tk,
                                                         causal, scale);
    else
        prefill_f32_kernel<128><<<grid, 256, 0, stream>>>(q, k, v, o, lse, Hq, Hkv, Tq, Tk,
                                                          causal, scale);
    return hipGetLastError();
}

}  // namespace attn
