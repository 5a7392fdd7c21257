// Paged decode attention with split-KV and a log-sum-exp combine.
//
// One query token per sequence reads the sequence's KV cache through a block
// table (paged attention, xhh.club summary, "how does paged attention manage
// the KV cache": fixed-size blocks, logical-to-physical table, logical order
// contiguous while physical placement is arbitrary).  The KV length is cut
// into chunks of split_tokens; each chunk yields an independent partial
// softmax state that is combined at the end (FlashDecoding, FlashDecoding++
// summary, wenjunhu.com/d/2311396.html, section 1).
//
// Decode is bound by reading the cache from HBM, so the kernel is organised
// around the loads:
//   * cache layout [page][kv_head][16][D]: one (page, kv head) tile is 4 KiB
//     contiguous (bf16, D = 128), read by one wavefront with four fully
//     coalesced 1 KiB load instructions for K and four for V;
//   * each wavefront walks every 4th page of its chunk and keeps the next
//     page's loads in flight while it computes the current one;
//   * the G = Hq/Hkv query heads that share a kv head are all served by the
//     one K/V tile that is loaded (grouped-query attention reads the cache
//     once, not G times);
//   * scores: a lane holds 8 (bf16) elements of one token row, so q.k is a
//     per-lane partial dot product (v_dot2_f32_bf16) finished by a 4-step
//     DPP reduction inside the 16-lane row;
//   * softmax state: each 16-lane row of a wavefront handles its own tokens
//     (token t of a page goes to row t % 4) with its own running max, sum and
//     output slice, so a page needs no cross-row communication at all.  The
//     4 rows x 4 wavefronts partial states are merged once, at the end of
//     the chunk, through LDS.
//   * the running max is only raised (and the state rescaled) when it grows
//     by more than 2^8; the exponentials are otherwise taken against the
//     stale max, which is exact up to rounding.
// A sequence that fits in one chunk is written straight to the output;
// otherwise each chunk writes (o / l, lse) in fp32 to the workspace and
// decode_combine_kernel merges them.
#include "common.h"
#include "kernels.h"

namespace attn {

namespace {

constexpr int kPage = 16;
constexpr float kRescaleThresh = 8.0f;

// Element access for the two storage types.
template <typename T>
struct Elem;
template <>
struct Elem<uint16_t> {
    static constexpr int kPerLoad = 8;  // elements per 16-byte load
    // dot of 8 bf16 q values with 8 bf16 k values, fp32 accumulation.  The
    // vector elements are copied to scalars before the bit cast: a bit cast
    // applied directly to an element of a vector reference was compiled into
    // a reuse of element 0.
    static __device__ __forceinline__ float dot(const u32x4& qv, const u32x4& kv, float acc) {
        const uint32_t qs[4] = {qv[0], qv[1], qv[2], qv[3]};
        const uint32_t ks[4] = {kv[0], kv[1], kv[2], kv[3]};
#pragma unroll
        for (int i = 0; i < 4; i++)
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qs[i]),
                                                  __builtin_bit_cast(bf16x2, ks[i]), acc, false);
        return acc;
    }
    static __device__ __forceinline__ float get(const u32x4& w, int e) {
        return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
    }
};
template <>
struct Elem<float> {
    static constexpr int kPerLoad = 4;
    static __device__ __forceinline__ float dot(const u32x4& qv, const u32x4& kv, float acc) {
#pragma unroll
        for (int i = 0; i < 4; i++) acc = fmaf(__uint_as_float(qv[i]), __uint_as_float(kv[i]), acc);
        return acc;
    }
    static __device__ __forceinline__ float get(const u32x4& w, int e) { return __uint_as_float(w[e]); }
};

// Sum over groups of LPT consecutive lanes (LPT in {8, 16, 32}); every lane
// of the group receives the total.  Within a 16-lane row this is DPP.
template <int LPT>
__device__ __forceinline__ float group_sum(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));  // quad [1,0,3,2]
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));  // quad [2,3,0,1]
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true)); // row half-mirror
    if (LPT >= 16)
        x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, true));  // row mirror
    if (LPT >= 32) x += __shfl_xor(x, 16);
    return x;
}

// (own value, value of lane ^ off) for off in {8, 16, 32}, in an order that
// is the same function of the unordered pair on both lanes' sides of every
// use below (all uses are symmetric: max, and sums of two products).
struct f32x2p {
    float a, b;
};
__device__ __forceinline__ f32x2p lane_pair(float x, int off) {
    if (off == 8) {  // swap the two halves of each 16-lane row
        return {x, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, true))};
    }
    if (off == 16) {
        auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        return {__uint_as_float(r[0]), __uint_as_float(r[1])};
    }
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

template <typename T, int D, int G>
struct DCfg {
    static constexpr int EPL = Elem<T>::kPerLoad;          // elements per lane per load
    static constexpr int LPT = D / EPL;                    // lanes per token row
    static constexpr int TPI = kWave / LPT;                // tokens per load instruction
    static constexpr int NLD = kPage / TPI;                // loads per page per tensor
};

template <typename T, int D, int G>
struct PageRegs {
    u32x4 k[DCfg<T, D, G>::NLD];
    u32x4 v[DCfg<T, D, G>::NLD];
};

template <typename T, int D, int G>
__device__ __forceinline__ void load_page(PageRegs<T, D, G>& r, const T* __restrict__ kp,
                                          const T* __restrict__ vp, size_t tile_off, int lane) {
    using C = DCfg<T, D, G>;
    const T* kt = kp + tile_off;
    const T* vt = vp + tile_off;
#pragma unroll
    for (int i = 0; i < C::NLD; i++) {
        r.k[i] = *(const u32x4*)(kt + (size_t)(i * kWave + lane) * C::EPL);
        r.v[i] = *(const u32x4*)(vt + (size_t)(i * kWave + lane) * C::EPL);
    }
}

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
    using C = DCfg<T, D, G>;
    using E = Elem<T>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int grp = lane / C::LPT;     // token group inside a load instruction
    const int col = lane % C::LPT;     // which EPL-element chunk of the row
    const int c = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    // lengths past the host bound are clamped, so no index leaves the planned
    // split range or the block-table row
    const int L_in = a.kv_lens ? a.kv_lens[b] : a.fixed_len;
    if (c == 0) check_len(L_in, a.max_len, a.err);
    const int L = min(L_in, a.max_len);
    const int nsplit = (L + a.split_tokens - 1) / a.split_tokens;
    const T* q = (const T*)a.q;

    if (L <= 0) {  // nothing to attend: O = 0, lse = -inf
        if (c == 0 && wave == 0) {
            for (int g = 0; g < G; g++) {
                const size_t row = (size_t)b * a.Hq + kvh * G + g;
                for (int d = lane; d < D; d += kWave) {
                    if (a.out_f32) ((float*)a.o)[row * D + d] = 0.f;
                    else ((uint16_t*)a.o)[row * D + d] = 0;
                }
                if (a.lse && lane == 0) a.lse[row] = -INFINITY;
            }
        }
        return;
    }
    if (c >= nsplit) return;

    const int tok0 = c * a.split_tokens;
    const int tok1 = min(L, tok0 + a.split_tokens);
    const int pg0 = tok0 / kPage, pg1 = (tok1 + kPage - 1) / kPage;
    const int32_t* table = a.block_table + (size_t)b * a.bt_stride;
    const size_t page_elems = (size_t)a.Hkv * kPage * D;
    const size_t head_off = (size_t)kvh * kPage * D;
    const float sl2 = a.scale * kLog2e;

    // this lane's query slices: q[h][col*EPL .. +EPL) for the G heads
    u32x4 qv[G];
#pragma unroll
    for (int g = 0; g < G; g++)
        qv[g] = *(const u32x4*)(q + ((size_t)b * a.Hq + kvh * G + g) * D + col * C::EPL);

    float m[G], l[G], acc[G][C::EPL];
#pragma unroll
    for (int g = 0; g < G; g++) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < C::EPL; e++) acc[g][e] = 0.f;
    }

    auto process = [&](const PageRegs<T, D, G>& r, int pg) {
        const int tbase = pg * kPage;
#pragma unroll
        for (int g = 0; g < G; g++) {
            float s[C::NLD];
            float smax = -INFINITY;
#pragma unroll
            for (int i = 0; i < C::NLD; i++) {
                const int t = tbase + i * C::TPI + grp;
                float x = group_sum<C::LPT>(E::dot(qv[g], r.k[i], 0.f));
                s[i] = (t < tok1) ? x : -INFINITY;
                smax = fmaxf(smax, s[i]);
            }
            smax = (smax == -INFINITY) ? -INFINITY : smax * sl2;
            const float m_new = fmaxf(m[g], smax);
            if (m_new > m[g] + kRescaleThresh) {
                const float alpha = fast_exp2(m[g] - m_new);
                l[g] *= alpha;
#pragma unroll
                for (int e = 0; e < C::EPL; e++) acc[g][e] *= alpha;
                m[g] = m_new;
            }
            const float m_eff = (m[g] == -INFINITY) ? 0.f : m[g];
#pragma unroll
            for (int i = 0; i < C::NLD; i++) {
                const float p = (s[i] == -INFINITY) ? 0.f : fast_exp2(__builtin_fmaf(s[i], sl2, -m_eff));
                l[g] += p;
#pragma unroll
                for (int e = 0; e < C::EPL; e++) acc[g][e] = fmaf(p, E::get(r.v[i], e), acc[g][e]);
            }
        }
    };

    // pages pg0 + wave, pg0 + wave + 4, ... with one page of loads in flight
    PageRegs<T, D, G> ra, rb;
    int pg = pg0 + wave;
    if (pg < pg1) load_page<T, D, G>(ra, (const T*)a.k_pages, (const T*)a.v_pages,
                                     (size_t)checked_page(table[pg], a.num_pages, a.err) * page_elems + head_off, lane);
    while (pg < pg1) {
        const int pn = pg + 4;
        if (pn < pg1) load_page<T, D, G>(rb, (const T*)a.k_pages, (const T*)a.v_pages,
                                         (size_t)checked_page(table[pn], a.num_pages, a.err) * page_elems + head_off, lane);
        process(ra, pg);
        pg = pn;
        if (pg >= pg1) break;
        const int pn2 = pg + 4;
        if (pn2 < pg1) load_page<T, D, G>(ra, (const T*)a.k_pages, (const T*)a.v_pages,
                                          (size_t)checked_page(table[pn2], a.num_pages, a.err) * page_elems + head_off, lane);
        process(rb, pg);
        pg = pn2;
    }

    // ---- merge the partial states: token groups of a wavefront by lane
    // swaps, then the 4 wavefronts through LDS ----------------------------
#pragma unroll
    for (int off = C::LPT; off < kWave; off <<= 1) {
#pragma unroll
        for (int g = 0; g < G; g++) {
            const f32x2p mp = lane_pair(m[g], off);
            const float M = fmaxf(mp.a, mp.b);
            const float wa = (mp.a == -INFINITY) ? 0.f : fast_exp2(mp.a - M);
            const float wb = (mp.b == -INFINITY) ? 0.f : fast_exp2(mp.b - M);
            const f32x2p lp = lane_pair(l[g], off);
            l[g] = wa * lp.a + wb * lp.b;
#pragma unroll
            for (int e = 0; e < C::EPL; e++) {
                const f32x2p ap = lane_pair(acc[g][e], off);
                acc[g][e] = wa * ap.a + wb * ap.b;
            }
            m[g] = M;
        }
    }
    __shared__ float s_m[G][4];
    __shared__ float s_l[G][4];
    __shared__ float s_o[G][4][D];
    if (grp == 0) {
#pragma unroll
        for (int g = 0; g < G; g++) {
            if (col == 0) {
                s_m[g][wave] = m[g];
                s_l[g][wave] = l[g];
            }
#pragma unroll
            for (int e = 0; e < C::EPL; e++) s_o[g][wave][col * C::EPL + e] = acc[g][e];
        }
    }
    __syncthreads();
    constexpr int NST = 4;

    // thread -> (head g, dim d); G*D <= 1024 outputs, 256 threads
    for (int idx = threadIdx.x; idx < G * D; idx += 256) {
        const int g = idx / D, d = idx % D;
        float M = -INFINITY;
        for (int j = 0; j < NST; j++) M = fmaxf(M, s_m[g][j]);
        float lt = 0.f, ot = 0.f;
        if (M != -INFINITY) {
            for (int j = 0; j < NST; j++) {
                const float w = (s_m[g][j] == -INFINITY) ? 0.f : fast_exp2(s_m[g][j] - M);
                lt = fmaf(w, s_l[g][j], lt);
                ot = fmaf(w, s_o[g][j][d], ot);
            }
        }
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        const float ov = ot * inv;
        const float lse = lt > 0.f ? (M + __log2f(lt)) * kLn2 : -INFINITY;
        const size_t row = (size_t)b * a.Hq + kvh * G + g;
        if (nsplit == 1) {
            if (a.out_f32) ((float*)a.o)[row * D + d] = ov;
            else ((uint16_t*)a.o)[row * D + d] = f32_to_bf16(ov);
            if (a.lse && d == 0) a.lse[row] = lse;
        } else {
            a.ws_o[(row * a.max_splits + c) * D + d] = ov;
            if (d == 0) a.ws_lse[row * a.max_splits + c] = lse;
        }
    }
}

// Combine the per-chunk states of every (sequence, head) row that was split:
//   lse = ln sum_c exp(lse_c),  o = sum_c exp(lse_c - lse) o_c.
// One 256-thread workgroup per row: D/4 lanes cover the row's dims with
// 16-byte loads, and the 256 / (D/4) lane groups take every NG-th chunk,
// each folding its chunks with a running max; the groups' states are then
// merged through LDS.  The many chunks of a few rows (small batches) are
// read by the whole workgroup at once instead of one wavefront in sequence.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
    constexpr int LPR = D / 4;       // lanes per row, 4 dims each
    constexpr int NG = 256 / LPR;    // chunk groups: 8 (D = 128) or 16 (D = 64)
    __shared__ float s_m[NG], s_l[NG];
    __shared__ f32x4 s_o[NG][LPR];
    const long row = blockIdx.x;
    const int b = (int)(row / a.Hq);
    const int grp = threadIdx.x / LPR, dl = threadIdx.x % LPR;
    const float* ls = a.ws_lse + row * a.max_splits;
    const f32x4* os = (const f32x4*)(a.ws_o + row * a.max_splits * D) + dl;
    // the group's first chunk is loaded together with the sequence length
    // (chunk grp < max_splits lies in the workspace; it is used only if the
    // sequence has that many chunks), so the two latencies overlap
    const bool pre = grp < a.max_splits;
    const float l0 = pre ? ls[grp] : -INFINITY;
    const f32x4 o0 = pre ? os[(size_t)grp * LPR] : f32x4{0.f, 0.f, 0.f, 0.f};
    const int L = min(a.kv_lens ? a.kv_lens[b] : a.fixed_len, a.max_len);
    // a cascade's rows hold prefix_slots prefix states before their own chunks'
    const int nsplit = a.prefix_slots + (L + a.split_tokens - 1) / a.split_tokens;
    // one chunk outside a cascade: written directly by the split kernel
    // (uniform per workgroup)
    if (nsplit <= 1 && a.prefix_slots == 0) return;
    float m = -INFINITY, l = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int c = grp; c < nsplit; c += NG) {
        const float lc = c == grp ? l0 : ls[c];
        const f32x4 oc = c == grp ? o0 : os[(size_t)c * LPR];
        const float mn = fmaxf(m, lc);
        const float sa = (m == -INFINITY) ? 0.f : expf(m - mn);
        const float sb = (lc == -INFINITY) ? 0.f : expf(lc - mn);
        l = fmaf(l, sa, sb);
#pragma unroll
        for (int e = 0; e < 4; e++) acc[e] = fmaf(acc[e], sa, sb * oc[e]);
        m = mn;
    }
    if (dl == 0) {
        s_m[grp] = m;
        s_l[grp] = l;
    }
    s_o[grp][dl] = acc;
    __syncthreads();
    if (grp != 0) return;
    float M = -INFINITY;
#pragma unroll
    for (int g = 0; g < NG; g++) M = fmaxf(M, s_m[g]);
    float lt = 0.f;
    f32x4 ot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < NG; g++) {
        const float w = (s_m[g] == -INFINITY) ? 0.f : expf(s_m[g] - M);
        lt = fmaf(w, s_l[g], lt);
        const f32x4 og = s_o[g][dl];
#pragma unroll
        for (int e = 0; e < 4; e++) ot[e] = fmaf(w, og[e], ot[e]);
    }
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (a.out_f32) {
        *(f32x4*)((float*)a.o + row * D + 4 * dl) = f32x4{ot[0] * inv, ot[1] * inv, ot[2] * inv, ot[3] * inv};
    } else {
        *(u32x2*)((uint16_t*)a.o + row * D + 4 * dl) =
            u32x2{(uint32_t)f32_to_bf16(ot[0] * inv) | ((uint32_t)f32_to_bf16(ot[1] * inv) << 16),
                  (uint32_t)f32_to_bf16(ot[2] * inv) | ((uint32_t)f32_to_bf16(ot[3] * inv) << 16)};
    }
    if (a.lse && dl == 0) a.lse[row] = lt > 0.f ? M + logf(lt) : -INFINITY;
}

hipError_t launch_combine(const DecodeArgs& a, hipStream_t stream) {
    const unsigned blocks = (unsigned)((long)a.B * a.Hq);
    if (a.D == 64) decode_combine_kernel<64><<<blocks, 256, 0, stream>>>(a);
    else decode_combine_kernel<128><<<blocks, 256, 0, stream>>>(a);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
    const dim3 grid(a.max_splits, a.Hkv, a.B);
    switch (a.Hq / a.Hkv) {
        case 1: decode_split_kernel<T, D, 1><<<grid, 256, 0, stream>>>(a); break;
        case 2: decode_split_kernel<T, D, 2><<<grid, 256, 0, stream>>>(a); break;
        case 4: decode_split_kernel<T, D, 4><<<grid, 256, 0, stream>>>(a); break;
        case 8: decode_split_kernel<T, D, 8><<<grid, 256, 0, stream>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.max_splits <= 1) return e;
    return launch_combine(a, stream);
}

}  // namespace

hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t stream) {
    return launch_combine(a, stream);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    if (a.in_f32) return a.D == 64 ? launch_typed<float, 64>(a, stream) : launch_typed<float, 128>(a, stream);
    return a.D == 64 ? launch_typed<uint16_t, 64>(a, stream) : launch_typed<uint16_t, 128>(a, stream);
}

}  // namespace attn
