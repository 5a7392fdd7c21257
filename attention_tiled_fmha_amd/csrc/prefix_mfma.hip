// Shared-prefix (cascade stage one) decode attention on gfx950 MFMA.
//
// Every request attends the same prefix, stored once in the paged cache
// (prefix sharing of KV blocks, xhh.club summary, "how does paged attention
// manage the KV cache"; the staged cascade of "FlashInfer kernel library",
// sections 2 and 4).  For one kv head the R requests x G grouped heads form
// N = R*G query rows that all meet the same keys, so the prefix stage is a
// small dense attention, [N rows] x [prefix keys], in which each prefix page
// is read from HBM once per kv head for all requests instead of once per
// request.
//
// The kernel is the paged decode kernel (decode_mfma.hip) with 32 query rows
// per item instead of G <= 16: per 16-token page a wavefront does, for two
// 16-row blocks j,
//   S_j^T = K Q_j^T      D/32 x v_mfma_f32_16x16x32_bf16
//   softmax(S_j)         per row over the page
//   O_j^T += V^T P_j^T   D/16 x v_mfma_f32_16x16x16_bf16
// where the K and V^T operand fragments, loaded once per page, serve both
// blocks.  Both blocks' scores are formed before either softmax, and one
// wave-uniform test decides a (rare) rescale of both, so the two MFMA chains
// and the two reductions overlap.  The register budget is held to 256 per
// lane (two waves per SIMD): the O accumulators then live in VGPRs, where
// the rescale multiplies them in place; with AGPR accumulators the compiler
// copied all of them out and back around the rescale branch on every page.  K is loaded straight into operand order and V transposed in
// registers, through per-page buffer descriptors that cover only the prefix
// (the tail of the last page reads zeros).  An FP8 cache is read with the
// paged decode kernel's FP8 layout: 16-byte K loads over a permuted
// contraction order (Q^T loaded in the same order) and, with D = 128, one
// 8-byte V load per token.
//
// An item is (chunk of the prefix, kv head, block of 32 rows); a persistent
// grid walks the items, kv head fastest, so the row blocks of one chunk and
// head run on one XCD and share its L2 copy of the pages.  The four
// wavefronts of a workgroup take every 4th page of the chunk and merge their
// states pairwise through LDS; the chunk's state goes to the workspace (or
// straight to the output when the prefix is one chunk) and the decode combine
// kernel folds the chunks.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace attn {

namespace {

constexpr int kPage = 16;
constexpr int kRB = 2;                   // 16-row query blocks per item
constexpr int kRows = 16 * kRB;          // 32 query rows per item
constexpr int kBufs = 2;                 // page buffers per wavefront
constexpr float kRescaleThresh = 8.0f;   // log2 units, as in the decode kernels
constexpr int kRsrcWord3 = 0x00020000;   // raw 32-bit data, no swizzle

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float max_xor16(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, bool FP8>
struct PrefixPage {
    u32x4 k[D / 32];          // K A operand of k-step s: token l % 16, dims 32s + 8(l/16) .. +7
    uint32_t v[4][D / 32];    // V: token 4(l/16) + t, dims 32c + 2(l%16), +1
};
template <int D>
struct PrefixPage<D, true> {
    u32x4 k[D / 64];          // K: 16 E4M3 bytes, token l%16, dims 16(l/16 + 4j) .. +15
    uint32_t v[4][D / 64];    // V: token 4(l/16) + t; D = 128: dims 8(l%16) + 4c .. +3,
                              // D = 64: dims 4(l%16) .. +3
};

// Two E4M3 bytes (the low or high half of w) -> two bf16, exactly.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// Head dimension of register r of O^T block i for lane group grp (row
// m = 4 grp + r of the block, held by lane m of the V operand): bf16 pages
// give blocks of even / odd dims of each 32-dim column, FP8 pages blocks of
// dims 4m + i%4 of each 64-dim column, or with D = 128 (V operand lane m
// holding dims 8m .. 8m + 7) dims 8m + i.
template <int D, bool FP8>
__device__ __forceinline__ int ot_dim(int i, int grp, int r) {
    if constexpr (!FP8) return 32 * (i >> 1) + 2 * (4 * grp + r) + (i & 1);
    return D == 128 ? 8 * (4 * grp + r) + 4 * (i >> 2) + (i & 3)
                    : 64 * (i >> 2) + 4 * (4 * grp + r) + (i & 3);
}

template <int D>
struct PrefixLds {
    static constexpr int STRIDE = D + 4;   // padded fp32 row
    static constexpr int SLOT = kRows * STRIDE;
    static constexpr size_t BYTES = (2 * SLOT + 4 * kRows) * sizeof(float);
};

template <int D, bool FP8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefix_mfma_kernel(PrefixArgs a) {
    constexpr int EB = FP8 ? 1 : 2;            // bytes per cached element
    constexpr int NBUF = FP8 ? 2 * kBufs : kBufs;   // as many bytes in flight for FP8
    constexpr int KS = D / 32;   // k-steps of S^T, and 32-dim V columns
    constexpr int NB = D / 16;   // 16-dim blocks of O^T
    using LD = PrefixLds<D>;
    extern __shared__ __attribute__((aligned(16))) float lds[];
    float* s_o = lds;                         // [2][kRows][STRIDE]
    float* s_m = lds + 2 * LD::SLOT;          // [2][kRows]
    float* s_l = s_m + 2 * kRows;             // [2][kRows]

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15, grp = lane >> 4;
    const int G = a.Hq / a.Hkv;
    const int N = a.R * G;                    // query rows of one kv head
    const int n_rb = (N + kRows - 1) / kRows;
    const int n_chunks = (a.prefix_len + a.chunk - 1) / a.chunk;
    // an FP8 cache holds k_scale * e4m3: the key scale joins the softmax scale,
    // the value scale multiplies the output (both are 1 for bf16)
    const float sl2 = a.scale * a.k_scale * kLog2e;
    const unsigned char* kbase = (const unsigned char*)a.k_pages;
    const unsigned char* vbase = (const unsigned char*)a.v_pages;
    const int voff_k = col * D * EB + 8 * EB * grp;
    const int voff_v = 4 * grp * D * EB + 4 * col;

    // query row n of kv head kvh: request n / G, head kvh*G + n % G
    auto qrow_of = [&](int kvh, int n) { return (size_t)(n / G) * a.Hq + kvh * G + n % G; };

    auto item = [&](const int c, const int kvh, const int rb) {
        const int tok0 = c * a.chunk;
        const int tok1 = min(a.prefix_len, tok0 + a.chunk);
        const int pg0 = tok0 / kPage;
        const int npg = (tok1 + kPage - 1) / kPage - pg0;   // <= 64 pages
        const int row0 = rb * kRows;

        // Q^T operands of the row blocks (zero past the last row)
        bf16x8 qf[kRB][KS];
#pragma unroll
        for (int j = 0; j < kRB; j++) {
            const int n = row0 + 16 * j + col;
            const uint16_t* qr = (const uint16_t*)a.q + qrow_of(kvh, min(n, N - 1)) * D;
#pragma unroll
            for (int s = 0; s < KS; s++) {
                // FP8: k-step s contracts the dims 16(grp + 4(s/2)) + 8(s%2) .. +7,
                // those of the half s%2 of the lane's 16-byte K load s/2
                const int d0 = FP8 ? 16 * (grp + 4 * (s >> 1)) + 8 * (s & 1) : 32 * s + 8 * grp;
                u32x4 w = *(const u32x4*)(qr + d0);
                if (n >= N) w = u32x4{0, 0, 0, 0};
                qf[j][s] = __builtin_bit_cast(bf16x8, w);
            }
        }
        const int tblv = lane < npg ? checked_page(a.pages[pg0 + lane], a.num_pages, a.err) : 0;

        auto load = [&](PrefixPage<D, FP8>& pb, int j) {
            const int pg = pg0 + j;
            const int phys = __builtin_amdgcn_readlane(tblv, min(j, npg - 1));
            const int bytes = __builtin_amdgcn_readfirstlane(max(0, min(kPage, tok1 - pg * kPage)) * D * EB);
            const size_t off = (((size_t)phys * a.Hkv + kvh) * kPage * D) * EB;
            const __amdgpu_buffer_rsrc_t rk =
                __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + off), (short)0, bytes, kRsrcWord3);
            const __amdgpu_buffer_rsrc_t rv =
                __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + off), (short)0, bytes, kRsrcWord3);
            if constexpr (FP8) {
#pragma unroll
                for (int jj = 0; jj < D / 64; jj++)
                    pb.k[jj] = __builtin_amdgcn_raw_buffer_load_b128(rk, col * D + 16 * (grp + 4 * jj), 0, 0);
#pragma unroll
                for (int t = 0; t < 4; t++) {
                    if constexpr (D == 128) {
                        // one 8-byte load: dims 8 col .. +7 of token 4 grp + t
                        const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(rv, (4 * grp + t) * D + 8 * col, 0, 0);
                        pb.v[t][0] = w[0];
                        pb.v[t][1] = w[1];
                    } else {
                        pb.v[t][0] = __builtin_amdgcn_raw_buffer_load_b32(rv, voff_v + t * D, 0, 0);
                    }
                }
            } else {
#pragma unroll
                for (int s = 0; s < KS; s++) pb.k[s] = __builtin_amdgcn_raw_buffer_load_b128(rk, voff_k + 64 * s, 0, 0);
#pragma unroll
                for (int t = 0; t < 4; t++)
#pragma unroll
                    for (int cc = 0; cc < KS; cc++)
                        pb.v[t][cc] = __builtin_amdgcn_raw_buffer_load_b32(rv, voff_v + t * D * 2 + 64 * cc, 0, 0);
            }
        };

        float m_run[kRB], l_run[kRB];
        f32x4 oacc[kRB][NB];
#pragma unroll
        for (int j = 0; j < kRB; j++) {
            m_run[j] = -INFINITY;
            l_run[j] = 0.f;
#pragma unroll
            for (int i = 0; i < NB; i++) oacc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

        auto compute = [&](const PrefixPage<D, FP8>& pb, int jp) {
            const int pg = pg0 + jp;
            // K A operands (FP8: bytes widened to bf16 once, for both row blocks)
            bf16x8 kf[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ks++) {
                if constexpr (FP8) {
                    const uint32_t w0 = pb.k[ks >> 1][2 * (ks & 1)], w1 = pb.k[ks >> 1][2 * (ks & 1) + 1];
                    kf[ks] = __builtin_bit_cast(bf16x8, u32x4{e4m3x2_to_bf16x2<false>(w0), e4m3x2_to_bf16x2<true>(w0),
                                                              e4m3x2_to_bf16x2<false>(w1), e4m3x2_to_bf16x2<true>(w1)});
                } else {
                    kf[ks] = __builtin_bit_cast(bf16x8, pb.k[ks]);
                }
            }
            // scores of every row block first: independent MFMA chains
            f32x4 s[kRB];
#pragma unroll
            for (int j = 0; j < kRB; j++) {
                s[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0], qf[j][0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
                for (int ks = 1; ks < KS; ks++)
                    s[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks], qf[j][ks], s[j], 0, 0, 0);
            }
            // s[j][r] is the score of token pg*16 + 4grp + r for row 16j + col
            if (pg * kPage + kPage > tok1) {
#pragma unroll
                for (int j = 0; j < kRB; j++)
#pragma unroll
                    for (int r = 0; r < 4; r++)
                        if (pg * kPage + 4 * grp + r >= tok1) s[j][r] = -INFINITY;
            }
            float mx[kRB];
#pragma unroll
            for (int j = 0; j < kRB; j++) mx[j] = fmaxf(fmaxf(s[j][0], s[j][1]), fmaxf(s[j][2], s[j][3]));
#pragma unroll
            for (int j = 0; j < kRB; j++) mx[j] = max_xor16(mx[j]);
#pragma unroll
            for (int j = 0; j < kRB; j++) mx[j] = max_xor32(mx[j]);
            bool grow = false;
#pragma unroll
            for (int j = 0; j < kRB; j++) {
                mx[j] = fmaxf(m_run[j], mx[j] * sl2);
                grow |= mx[j] > m_run[j] + kRescaleThresh;
            }
            if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
                for (int j = 0; j < kRB; j++) {
                    const float alpha = (mx[j] == -INFINITY) ? 1.f : fast_exp2(m_run[j] - mx[j]);
                    l_run[j] *= alpha;
#pragma unroll
                    for (int i = 0; i < NB; i++) oacc[j][i] *= alpha;
                    m_run[j] = mx[j];
                }
            }
            s16x4 pt[kRB];
#pragma unroll
            for (int j = 0; j < kRB; j++) {
                const float m_eff = (m_run[j] == -INFINITY) ? 0.f : m_run[j];
                float p[4];
#pragma unroll
                for (int r = 0; r < 4; r++) p[r] = fast_exp2(__builtin_fmaf(s[j][r], sl2, -m_eff));
                const uint32_t p01 = pack_bf16x2(p[0], p[1]), p23 = pack_bf16x2(p[2], p[3]);
                // the row sum adds the bf16-rounded P that meets V
                l_run[j] += (bf16_lo(p01) + bf16_hi(p01)) + (bf16_lo(p23) + bf16_hi(p23));
                pt[j] = __builtin_bit_cast(s16x4, u32x2{p01, p23});
            }
            if constexpr (FP8) {
                // per 64-dim column c: block 4c + i gathers dim offset i of the 4 tokens
#pragma unroll
                for (int cc = 0; cc < D / 64; cc++) {
                    uint32_t lo[4], hi[4];
#pragma unroll
                    for (int t = 0; t < 4; t++) {
                        lo[t] = e4m3x2_to_bf16x2<false>(pb.v[t][cc]);   // dims +0, +1
                        hi[t] = e4m3x2_to_bf16x2<true>(pb.v[t][cc]);    // dims +2, +3
                    }
                    s16x4 av[4];
                    av[0] = __builtin_bit_cast(s16x4, u32x2{__builtin_amdgcn_perm(lo[1], lo[0], 0x05040100u),
                                                            __builtin_amdgcn_perm(lo[3], lo[2], 0x05040100u)});
                    av[1] = __builtin_bit_cast(s16x4, u32x2{__builtin_amdgcn_perm(lo[1], lo[0], 0x07060302u),
                                                            __builtin_amdgcn_perm(lo[3], lo[2], 0x07060302u)});
                    av[2] = __builtin_bit_cast(s16x4, u32x2{__builtin_amdgcn_perm(hi[1], hi[0], 0x05040100u),
                                                            __builtin_amdgcn_perm(hi[3], hi[2], 0x05040100u)});
                    av[3] = __builtin_bit_cast(s16x4, u32x2{__builtin_amdgcn_perm(hi[1], hi[0], 0x07060302u),
                                                            __builtin_amdgcn_perm(hi[3], hi[2], 0x07060302u)});
#pragma unroll
                    for (int j = 0; j < kRB; j++)
#pragma unroll
                        for (int i = 0; i < 4; i++)
                            oacc[j][4 * cc + i] =
                                __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av[i], pt[j], oacc[j][4 * cc + i], 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int cc = 0; cc < KS; cc++) {
                    const uint32_t v0 = pb.v[0][cc], v1 = pb.v[1][cc], v2 = pb.v[2][cc], v3 = pb.v[3][cc];
                    const s16x4 ae = __builtin_bit_cast(s16x4, u32x2{__builtin_amdgcn_perm(v1, v0, 0x05040100u),
                                                                     __builtin_amdgcn_perm(v3, v2, 0x05040100u)});
                    const s16x4 ao = __builtin_bit_cast(s16x4, u32x2{__builtin_amdgcn_perm(v1, v0, 0x07060302u),
                                                                     __builtin_amdgcn_perm(v3, v2, 0x07060302u)});
#pragma unroll
                    for (int j = 0; j < kRB; j++) {
                        oacc[j][2 * cc] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ae, pt[j], oacc[j][2 * cc], 0, 0, 0);
                        oacc[j][2 * cc + 1] =
                            __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ao, pt[j], oacc[j][2 * cc + 1], 0, 0, 0);
                    }
                }
            }
        };

        // pages j = wave, wave + 4, ... with the next kBufs - 1 pages' loads in
        // flight (one workgroup per CU: the depth sets the bytes in flight);
        // the loads are unconditional so that each wait covers exactly one page
        // The page count is padded to a multiple of kBufs: a page past the
        // chunk reads zeros and is masked out, so it adds exactly nothing, and
        // the loop body has no early exit between its loads.
        const int nj = npg > wave ? (npg - wave + 3) / 4 : 0;
        const int nj_pad = (nj + NBUF - 1) / NBUF * NBUF;
        PrefixPage<D, FP8> buf[NBUF];
#pragma unroll
        for (int u = 0; u < NBUF - 1; u++) load(buf[u], wave + 4 * u);
        for (int n = 0; n < nj_pad; n += NBUF) {
#pragma unroll
            for (int u = 0; u < NBUF; u++) {
                load(buf[(u + NBUF - 1) % NBUF], wave + 4 * (n + u + NBUF - 1));
                compute(buf[u], wave + 4 * (n + u));
            }
        }
#pragma unroll
        for (int j = 0; j < kRB; j++) l_run[j] = sum_xor32(sum_xor16(l_run[j]));

        // ---- merge the four wavefronts: 2,3 into 0,1, then 1 into 0 --------
        // O^T block i of row block j, register r: row 16j + col, dim ot_dim
        auto put = [&](int slot) {
            float* o = s_o + slot * LD::SLOT;
#pragma unroll
            for (int j = 0; j < kRB; j++) {
                if (grp == 0) {
                    s_m[slot * kRows + 16 * j + col] = m_run[j];
                    s_l[slot * kRows + 16 * j + col] = l_run[j];
                }
#pragma unroll
                for (int i = 0; i < NB; i++)
#pragma unroll
                    for (int r = 0; r < 4; r++)
                        o[(16 * j + col) * LD::STRIDE + ot_dim<D, FP8>(i, grp, r)] = oacc[j][i][r];
            }
        };
        auto take = [&](int slot) {
            const float* o = s_o + slot * LD::SLOT;
#pragma unroll
            for (int j = 0; j < kRB; j++) {
                const float mb = s_m[slot * kRows + 16 * j + col], lb = s_l[slot * kRows + 16 * j + col];
                const float M = fmaxf(m_run[j], mb);
                const float wa = (m_run[j] == -INFINITY) ? 0.f : fast_exp2(m_run[j] - M);
                const float wb = (mb == -INFINITY) ? 0.f : fast_exp2(mb - M);
                l_run[j] = wa * l_run[j] + wb * lb;
                m_run[j] = M;
#pragma unroll
                for (int i = 0; i < NB; i++)
#pragma unroll
                    for (int r = 0; r < 4; r++)
                        oacc[j][i][r] = wa * oacc[j][i][r] +
                                        wb * o[(16 * j + col) * LD::STRIDE + ot_dim<D, FP8>(i, grp, r)];
            }
        };
        if (wave >= 2) put(wave - 2);
        __syncthreads();
        if (wave < 2) take(wave);
        __syncthreads();
        if (wave == 1) put(0);
        __syncthreads();
        if (wave == 0) {
            take(0);
            // normalised rows to slot 0 in row-major order, lse to s_m
            float* o = s_o;
#pragma unroll
            for (int j = 0; j < kRB; j++) {
                const float inv = l_run[j] > 0.f ? a.v_scale / l_run[j] : 0.f;
                if (grp == 0)
                    s_m[16 * j + col] = l_run[j] > 0.f ? (m_run[j] + __log2f(l_run[j])) * kLn2 : -INFINITY;
#pragma unroll
                for (int i = 0; i < NB; i++)
#pragma unroll
                    for (int r = 0; r < 4; r++)
                        o[(16 * j + col) * LD::STRIDE + ot_dim<D, FP8>(i, grp, r)] = oacc[j][i][r] * inv;
            }
        }
        __syncthreads();
        // all threads: rows out, 4 dims per thread
        for (int idx = threadIdx.x; idx < kRows * (D / 4); idx += 256) {
            const int rr = idx / (D / 4), d0 = 4 * (idx % (D / 4));
            const int n = row0 + rr;
            if (n >= N) continue;
            const size_t row = qrow_of(kvh, n);
            const f32x4 v = *(const f32x4*)(s_o + rr * LD::STRIDE + d0);
            if (n_chunks > 1 || a.ws_slots > 0) {
                const size_t slot = row * (a.ws_slots > 0 ? a.ws_slots : n_chunks) + c;
                *(f32x4*)(a.ws_o + slot * D + d0) = v;
                if (d0 == 0) a.ws_lse[slot] = s_m[rr];
            } else {
                if (a.out_f32) *(f32x4*)((float*)a.o + row * D + d0) = v;
                else *(u32x2*)((uint16_t*)a.o + row * D + d0) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                if (a.lse && d0 == 0) a.lse[row] = s_m[rr];
            }
        }
        __syncthreads();   // the LDS slots are rewritten by the next item
    };

    const long n_items = (long)n_chunks * a.Hkv * n_rb;
    for (long n = blockIdx.x; n < n_items; n += gridDim.x) {
        const int kvh = (int)(n % a.Hkv);
        const long r = n / a.Hkv;
        item((int)(r / n_rb), kvh, (int)(r % n_rb));
    }
}

}  // namespace

size_t prefix_lds_bytes(int D) {
    return D == 64 ? PrefixLds<64>::BYTES : PrefixLds<128>::BYTES;
}

hipError_t launch_prefix(const PrefixArgs& a, hipStream_t stream) {
    const int N = a.R * (a.Hq / a.Hkv);
    const long n_items = (long)((a.prefix_len + a.chunk - 1) / a.chunk) * a.Hkv * ((N + kRows - 1) / kRows);
    const dim3 grid((unsigned)std::min<long>(n_items, 4096));
    const size_t lds = prefix_lds_bytes(a.D);
    auto go = [&](auto kern) {
        hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        kern<<<grid, 256, lds, stream>>>(a);
    };
    if (a.in_fp8)
        a.D == 64 ? go(prefix_mfma_kernel<64, true>) : go(prefix_mfma_kernel<128, true>);
    else
        a.D == 64 ? go(prefix_mfma_kernel<64, false>) : go(prefix_mfma_kernel<128, false>);
    return hipGetLastError();
}

}  // namespace attn
