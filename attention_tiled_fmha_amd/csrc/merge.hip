// Merge of two partial attention states (o_a, lse_a) (+) (o_b, lse_b) in place
// into a: the combining step of split / cascade attention.
//
//   M = max(lse_a, lse_b);  w_x = exp(lse_x - M);
//   lse = M + ln(w_a + w_b);  o = (w_a o_a + w_b o_b) / (w_a + w_b)
//
// A side with lse = -inf is empty: its weight is 0 and its o is never read
// into the sum, so whatever it holds (even NaN) cannot leak.
//
// Bandwidth-trivial: one thread per 4 consecutive elements of a row; the
// D/4 threads of a row sit in one wavefront, so every lane has read lse_a
// before the row's first lane overwrites it.
#include "common.h"
#include "kernels.h"

namespace attn {

template <typename T>
struct Quad;
template <>
struct Quad<float> {
    static __device__ __forceinline__ f32x4 load(const float* p) { return *(const f32x4*)p; }
    static __device__ __forceinline__ void store(float* p, f32x4 v) { *(f32x4*)p = v; }
};
template <>
struct Quad<uint16_t> {
    static __device__ __forceinline__ f32x4 load(const uint16_t* p) {
        u32x2 w = *(const u32x2*)p;
        return f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
    }
    static __device__ __forceinline__ void store(uint16_t* p, f32x4 v) {
        *(u32x2*)p = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
};

template <typename T>
__global__ __launch_bounds__(256) void merge_states_kernel(T* o_a, float* lse_a, const T* o_b,
                                                           const float* lse_b, int rows, int D) {
    // o_b / lse_b may alias o_a / lse_a exactly: no __restrict__ here.
    const int per_row = D >> 2;
    const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long row = gid / per_row;
    const int c = (int)(gid - row * per_row);
    if (row >= rows) return;
    // all four loads are issued before any of them is used (one memory
    // latency per thread, not two)
    const size_t off = (size_t)row * D + 4 * c;
    const float la = lse_a[row], lb = lse_b[row];
    const f32x4 oa = Quad<T>::load(o_a + off), ob = Quad<T>::load(o_b + off);
    const float M = fmaxf(la, lb);
    float wa = 0.f, wb = 0.f, lse = -INFINITY;
    if (M != -INFINITY) {
        wa = expf(la - M);
        wb = expf(lb - M);
        lse = M + logf(wa + wb);
    }
    const float inv = (wa + wb) > 0.f ? 1.f / (wa + wb) : 0.f;
    f32x4 r;
#pragma unroll
    for (int e = 0; e < 4; e++)   // selects, so an empty side's o (even NaN) adds nothing
        r[e] = (wa > 0.f ? wa * oa[e] : 0.f) + (wb > 0.f ? wb * ob[e] : 0.f);
    Quad<T>::store(o_a + off, r * inv);
    if (c == 0) lse_a[row] = lse;
}

hipError_t launch_merge_states(void* o_a, float* lse_a, const void* o_b, const float* lse_b,
                               int rows, int D, bool f32, hipStream_t stream) {
    const long threads = (long)rows * (D / 4);
    const int blocks = (int)((threads + 255) / 256);
    if (f32)
        merge_states_kernel<float><<<blocks, 256, 0, stream>>>(
            (float*)o_a, lse_a, (const float*)o_b, lse_b, rows, D);
    else
        merge_states_kernel<uint16_t><<<blocks, 256, 0, stream>>>(
            (uint16_t*)o_a, lse_a, (const uint16_t*)o_b, lse_b, rows, D);
    return hipGetLastError();
}

}  // namespace attn
