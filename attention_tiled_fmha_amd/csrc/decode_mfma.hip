// Paged split-KV decode on gfx950 MFMA (bf16 cache), for any number G <= 16
// of query heads per kv head.
//
// Same problem and work split as decode.hip: one query token per sequence,
// its KV cache read through a block table (paged attention, xhh.club summary,
// "how does paged attention manage the KV cache"), the KV length cut into
// chunks whose partial softmax states are merged with their log-sum-exp
// (FlashDecoding++ summary, wenjunhu.com/d/2311396.html, section 1).  The
// cache layout is [page][kv_head][16][D].
//
// Per 16-token page a wavefront does the two contractions on the matrix core
// with the G query heads as the (zero-padded) 16-wide N dimension:
//   S^T = K Q^T     D/32 x v_mfma_f32_16x16x32_bf16.  K is loaded straight
//                   into A-operand order (lane l: token l % 16, dims
//                   32s + 8(l/16) .. +7) and Q^T is the B operand, loaded once.
//                   The accumulator gives lane l the scores of head l % 16 for
//                   tokens 4(l/16) .. +3.
//   softmax         per head over the page (lane-local max of 4, then two lane
//                   swaps); P rounded to bf16 is already the B operand of PV.
//   O^T += V^T P^T  D/16 x v_mfma_f32_16x16x16_bf16.  Per 32-dim column c a
//                   lane loads one dword (2 dims) of each of 4 consecutive
//                   tokens; two v_perm give the A operands of two 16-dim
//                   blocks, block 2c holding the even and block 2c+1 the odd
//                   dims of 32c .. 32c+31.
// so the VALU work per page no longer grows with G (the head loop of the
// vector kernel did q.k, the reductions and the exponentials per head).
//
// Loads: one raw buffer descriptor per page covers only the page's valid
// tokens, so the tail of the last page reads zeros (and cannot feed garbage
// into the MFMAs) and out-of-range prefetches cost nothing.  Each wavefront
// walks every 4th page of the chunk with the next page's loads in flight.
// The chunk's block-table entries (a chunk is at most 64 pages) are read
// once into a register and picked with v_readlane.  The four wavefronts'
// states are merged through LDS at the end, as in the vector kernel.
//
// An FP8 (E4M3) cache is widened to bf16 in registers, exactly.  Its loads
// are wider than the bf16 layout above would give: K is read as one 16-byte
// load per lane per 64 dims (token l % 16, dims 16(l/16 + 4j) .. +15) and
// S^T contracts the dims in that order (k-step s takes half s % 2 of load
// s / 2; Q^T is loaded in the same order), and with D = 128 V is read as one
// 8-byte load per token (dims 8(l % 16) .. +7 of token 4(l/16) + t), whose
// two words give four 16-dim blocks each.  Against 8-byte K and 4-byte V
// loads this took the FP8 GQA workload from 614 to 572 us and MHA from 218
// to 210.
//
// The grid is persistent: a fixed number of workgroups walks the
// (chunk, kv head, sequence) items chunk-major.  The grid over the longest
// sequence holds many empty chunks (a batch of mixed lengths); as separate
// workgroups each of them cost a launch and a cold length load, here a few
// scalar instructions.  With chunks of at most 512 tokens an item holds two
// consecutive chunks of one (sequence, kv head), four over an FP8 cache: the
// page pipeline runs on across the chunk boundaries, which saves one pipeline
// start per chunk after the first (two chunks: measured 2-3% on 512-token
// chunks of bf16, 4-5% of FP8; four FP8 chunks another 4%); each chunk still
// gets its own partial state.
#include "common.h"
#include "kernels.h"

#include <algorithm>
#include <type_traits>

namespace attn {

namespace {

constexpr int kPage = 16;
constexpr int kMaxG = 16;
constexpr float kRescaleThresh = 8.0f;   // log2 units, as in the vector kernel
constexpr float kUnifiedWindow = 60.0f;  // |max scaled score - phi| bound of the unified max
constexpr int kRsrcWord3 = 0x00020000;   // raw 32-bit data, no swizzle

typedef short s16x4 __attribute__((ext_vector_type(4)));

// One page's operands in flight, per lane.
template <int D, bool FP8>
struct PageBuf {
    u32x4 k[D / 32];          // K A operand of k-step s (8 bf16)
    uint32_t v[4][D / 32];    // V: token 4(l/16) + t, dims 32c + 2(l%16), +1
};
template <int D>
struct PageBuf<D, true> {
    u32x4 k[D / 64];          // K: 16 E4M3 bytes, token l%16, dims 16(l/16 + 4j) .. +15
    uint32_t v[4][D / 64];    // V: token 4(l/16) + t; D = 128: dims 8(l%16) + 4c .. +3,
                              // D = 64: dims 4(l%16) .. +3
};

// Two E4M3 bytes (the low or high half of w) -> two bf16, exactly (every
// E4M3 value is a bf16 value; the conversion's scale is 1).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// (own value, value of lane ^ 16 or lane ^ 32); only used symmetrically
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

// Chunks per work item: consecutive chunks of one (sequence, kv head) share
// an item when each chunk's pages split evenly over the wavefronts' unit
// pairs and the item fits two 64-entry table windows; the page pipeline then
// runs on across the chunk boundaries.  bf16 items hold two chunks, FP8
// items (half the bytes per page, so the per-item start weighs twice as
// much) four.  The unified-max path keeps one.
__host__ __device__ inline int chunks_per_item(const DecodeArgs& a, bool fp8) {
    const int unit = fp8 ? 2 : 1;   // pages per unit
    return (!a.unified && a.split_tokens <= 32 * kPage && a.split_tokens % (8 * kPage * unit) == 0)
               ? (fp8 ? 4 : 2) : 1;
}

template <int D, bool FP8>
__global__ __launch_bounds__(256) void decode_mfma_kernel(DecodeArgs a) {
    constexpr int EB = FP8 ? 1 : 2;   // bytes per cached element
    constexpr int KS = D / 32;   // k-steps of S^T, and 32-dim V columns
    constexpr int NB = D / 16;   // 16-dim blocks of O^T
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15, grp = lane >> 4;
    const int G = a.Hq / a.Hkv;
    // the wavefronts' published states, two sets: an item's two chunks are
    // published one after the other and merged together at its end
    __shared__ float s_m[2][4][kMaxG];
    __shared__ float s_l[2][4][kMaxG];
    __shared__ float s_x[4][kMaxG];     // unified max: largest raw score per row
    __shared__ __attribute__((aligned(16))) float s_o[2][4][kMaxG][D];
    const float phi_l2 = a.phi * kLog2e;
    const int cpi = chunks_per_item(a, FP8);
    // in a cascade the first prefix_slots workspace slots of every row hold the
    // prefix stage's chunk states: the sequence's chunks follow them, and every
    // chunk (also a sequence's only one) goes to the workspace
    const int slot0 = a.prefix_slots;
    const bool cascade = slot0 > 0;
    auto item = [&](const int ci, const int kvh, const int b) {
        // lengths past the host bound are clamped, so no index leaves the planned
        // split range or the block-table row
        const int L_in = a.kv_lens ? a.kv_lens[b] : a.fixed_len;
        if (ci == 0) check_len(L_in, a.max_len, a.err);
        const int L = min(L_in, a.max_len);
        const int nsplit = (L + a.split_tokens - 1) / a.split_tokens;

        if (L <= 0) {  // nothing to attend: O = 0, lse = -inf (a cascade's
                       // combine merges the prefix slots alone)
            if (!cascade && ci == 0 && wave == 0) {
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
        const int c = ci * cpi;                   // the item's first chunk
        if (c >= nsplit) return;
        const int ncs = min(cpi, nsplit - c);     // its chunks (the first of two is full)

        const int tok0 = c * a.split_tokens;
        const int tok1 = min(L, tok0 + ncs * a.split_tokens);
        const int pg0 = tok0 / kPage, pg1 = (tok1 + kPage - 1) / kPage;
        const int npg = pg1 - pg0;
        const int32_t* table = a.block_table + (size_t)b * a.bt_stride;
        // an FP8 cache holds k_scale * e4m3: the key scale joins the softmax
        // scale, the value scale multiplies the output
        const float sl2 = a.scale * a.k_scale * kLog2e;
        const unsigned char* kbase = (const unsigned char*)a.k_pages;
        const unsigned char* vbase = (const unsigned char*)a.v_pages;

        // Q^T (B operand): head col (zero for col >= G), dims 32s + 8grp .. +7
        bf16x8 qf[KS];
        {
            const uint16_t* qrow = (const uint16_t*)a.q + ((size_t)b * a.Hq + kvh * G + min(col, G - 1)) * D;
    #pragma unroll
            for (int s = 0; s < KS; s++) {
                // FP8: k-step s contracts the dims 16(grp + 4(s/2)) + 8(s%2) .. +7,
                // those of the half s%2 of the lane's 16-byte K load s/2
                const int d0 = FP8 ? 16 * (grp + 4 * (s >> 1)) + 8 * (s & 1) : 32 * s + 8 * grp;
                u32x4 w = *(const u32x4*)(qrow + d0);
                if (col >= G) w = u32x4{0, 0, 0, 0};
                qf[s] = __builtin_bit_cast(bf16x8, w);
            }
        }

        // the item's block-table entries (at most 128 pages): entries pg0 + lane
        // and pg0 + 64 + lane, picked with v_readlane
        const int tblv = lane < npg ? checked_page(table[pg0 + lane], a.num_pages, a.err) : 0;
        const int tblv2 = lane + 64 < npg ? checked_page(table[pg0 + 64 + lane], a.num_pages, a.err) : 0;
        auto phys_of = [&](int j) { return __builtin_amdgcn_readlane(j < 64 ? tblv : tblv2, j & 63); };

        // byte offsets of this lane's K and V elements in a page tile
        const int voff_k = col * D * EB + 8 * EB * grp;
        const int voff_v = 4 * grp * D * EB + 4 * col;
        // page j of the chunk; past the chunk the descriptor is empty and the
        // loads return zeros without touching memory
        auto load = [&](PageBuf<D, FP8>& pb, int j) {
            const int pg = pg0 + j;
            const int phys = phys_of(min(j, npg - 1));
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
                for (int t = 0; t < 4; t++)
    #pragma unroll
                    for (int cc = 0; cc < D / 64; cc++)
                        if constexpr (D == 128) {
                            // one 8-byte load: dims 8 col .. +7 of token 4 grp + t
                            if (cc == 0) {
                                const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(rv, (4 * grp + t) * D + 8 * col, 0, 0);
                                pb.v[t][0] = w[0];
                                pb.v[t][1] = w[1];
                            }
                        } else {
                            pb.v[t][cc] = __builtin_amdgcn_raw_buffer_load_b32(rv, voff_v + t * D + 64 * cc, 0, 0);
                        }
            } else {
    #pragma unroll
                for (int s = 0; s < KS; s++) pb.k[s] = __builtin_amdgcn_raw_buffer_load_b128(rk, voff_k + 64 * s, 0, 0);
    #pragma unroll
                for (int t = 0; t < 4; t++)
    #pragma unroll
                    for (int cc = 0; cc < D / 32; cc++)
                        pb.v[t][cc] = __builtin_amdgcn_raw_buffer_load_b32(rv, voff_v + t * D * 2 + 64 * cc, 0, 0);
            }
        };

        // merge the four wavefronts' states published in set `set` and write
        // chunk cc's result (straight to the output when the sequence is one
        // chunk); the caller synchronises before the set is published again
        auto finish = [&](int cc, int set) {
            // a thread per 4 consecutive dims of a row: the four wavefronts'
            // weights once, then 16-byte LDS reads and global writes
            for (int idx = threadIdx.x; idx < G * (D / 4); idx += 256) {
                const int g = idx / (D / 4), d0 = 4 * (idx % (D / 4));
                float M = -INFINITY;
                for (int w = 0; w < 4; w++) M = fmaxf(M, s_m[set][w][g]);
                float lt = 0.f;
                f32x4 ot = {0.f, 0.f, 0.f, 0.f};
                if (M != -INFINITY) {
                    for (int w = 0; w < 4; w++) {
                        const float sm = s_m[set][w][g];
                        const float wt = (sm == -INFINITY) ? 0.f : fast_exp2(sm - M);
                        lt = fmaf(wt, s_l[set][w][g], lt);
                        const f32x4 ow = *(const f32x4*)&s_o[set][w][g][d0];
#pragma unroll
                        for (int e = 0; e < 4; e++) ot[e] = fmaf(wt, ow[e], ot[e]);
                    }
                }
                const float inv = lt > 0.f ? a.v_scale / lt : 0.f;
                f32x4 ov;
#pragma unroll
                for (int e = 0; e < 4; e++) ov[e] = ot[e] * inv;
                const float lse = lt > 0.f ? (M + __log2f(lt)) * kLn2 : -INFINITY;
                const size_t row = (size_t)b * a.Hq + kvh * G + g;
                if (nsplit == 1 && !cascade) {
                    if (a.out_f32) *(f32x4*)((float*)a.o + row * D + d0) = ov;
                    else *(u32x2*)((uint16_t*)a.o + row * D + d0) =
                             u32x2{pack_bf16x2(ov[0], ov[1]), pack_bf16x2(ov[2], ov[3])};
                    if (a.lse && d0 == 0) a.lse[row] = lse;
                } else {
                    *(f32x4*)(a.ws_o + (row * a.max_splits + slot0 + cc) * D + d0) = ov;
                    if (d0 == 0) a.ws_lse[row * a.max_splits + slot0 + cc] = lse;
                }
            }
        };

        float m_run = -INFINITY, l_run = 0.f, smax = -INFINITY;
        f32x4 oacc[NB];

        // One pass over the chunk's pages, with the result published to LDS.
        // EXACT: online softmax against the running max (raised lazily).  Else
        // the unified-max softmax: every exponential is taken against the
        // caller's phi, with no running max, no rescale and no cross-lane max;
        // smax only tracks the lane's largest raw score, so that a row leaving
        // the safe window around phi can be detected after the pass.
        auto pass = [&](auto EXACT) {
            constexpr bool exact = decltype(EXACT)::value;
            m_run = exact ? -INFINITY : phi_l2;
            l_run = 0.f;
            smax = -INFINITY;
    #pragma unroll
            for (int i = 0; i < NB; i++) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

            auto compute = [&](const PageBuf<D, FP8>& pb, int j) {
                const int pg = pg0 + j;
                // K A operand of k-step ks (FP8: 8 bytes widened to bf16)
                auto kop = [&](int ks) -> bf16x8 {
                    if constexpr (FP8) {
                        const uint32_t w0 = pb.k[ks >> 1][2 * (ks & 1)], w1 = pb.k[ks >> 1][2 * (ks & 1) + 1];
                        return __builtin_bit_cast(bf16x8, u32x4{e4m3x2_to_bf16x2<false>(w0), e4m3x2_to_bf16x2<true>(w0),
                                                                e4m3x2_to_bf16x2<false>(w1), e4m3x2_to_bf16x2<true>(w1)});
                    } else {
                        return __builtin_bit_cast(bf16x8, pb.k[ks]);
                    }
                };
                f32x4 s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop(0), qf[0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    #pragma unroll
                for (int ks = 1; ks < KS; ks++)
                    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop(ks), qf[ks], s, 0, 0, 0);
                // s[r] is the score of token pg*16 + 4grp + r for head col
                if (pg * kPage + kPage > tok1) {
    #pragma unroll
                    for (int r = 0; r < 4; r++)
                        if (pg * kPage + 4 * grp + r >= tok1) s[r] = -INFINITY;
                }
                float m_eff;
                if (exact) {
                    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
                    mx = max_xor32(max_xor16(mx));
                    const float m_new = fmaxf(m_run, mx * sl2);
                    if (__builtin_amdgcn_ballot_w64(m_new > m_run + kRescaleThresh)) {
                        const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
                        l_run *= alpha;
    #pragma unroll
                        for (int i = 0; i < NB; i++) oacc[i] *= alpha;
                        m_run = m_new;
                    }
                    m_eff = (m_run == -INFINITY) ? 0.f : m_run;
                } else {
                    smax = fmaxf(smax, fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
                    m_eff = phi_l2;
                }
                float p[4];
    #pragma unroll
                for (int r = 0; r < 4; r++) p[r] = fast_exp2(__builtin_fmaf(s[r], sl2, -m_eff));
                const uint32_t p01 = pack_bf16x2(p[0], p[1]), p23 = pack_bf16x2(p[2], p[3]);
                // the row sum adds the bf16-rounded P that meets V
                l_run += (bf16_lo(p01) + bf16_hi(p01)) + (bf16_lo(p23) + bf16_hi(p23));
                const s16x4 pt = __builtin_bit_cast(s16x4, u32x2{p01, p23});
                if constexpr (FP8) {
                    // per 64-dim column c: lane holds dims 64c + 4(l%16) + {0..3} of its 4
                    // tokens; block 4c + i gathers dim offset i of the 4 tokens
    #pragma unroll
                    for (int cc = 0; cc < D / 64; cc++) {
                        uint32_t lo[4], hi[4];
    #pragma unroll
                        for (int t = 0; t < 4; t++) {
                            lo[t] = e4m3x2_to_bf16x2<false>(pb.v[t][cc]);   // dims +0, +1
                            hi[t] = e4m3x2_to_bf16x2<true>(pb.v[t][cc]);    // dims +2, +3
                        }
                        const s16x4 a0 = __builtin_bit_cast(s16x4, u32x2{__builtin_amdgcn_perm(lo[1], lo[0], 0x05040100u),
                                                                         __builtin_amdgcn_perm(lo[3], lo[2], 0x05040100u)});
                        const s16x4 a1 = __builtin_bit_cast(s16x4, u32x2{__builtin_amdgcn_perm(lo[1], lo[0], 0x07060302u),
                                                                         __builtin_amdgcn_perm(lo[3], lo[2], 0x07060302u)});
                        const s16x4 a2 = __builtin_bit_cast(s16x4, u32x2{__builtin_amdgcn_perm(hi[1], hi[0], 0x05040100u),
                                                                         __builtin_amdgcn_perm(hi[3], hi[2], 0x05040100u)});
                        const s16x4 a3 = __builtin_bit_cast(s16x4, u32x2{__builtin_amdgcn_perm(hi[1], hi[0], 0x07060302u),
                                                                         __builtin_amdgcn_perm(hi[3], hi[2], 0x07060302u)});
                        oacc[4 * cc] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a0, pt, oacc[4 * cc], 0, 0, 0);
                        oacc[4 * cc + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a1, pt, oacc[4 * cc + 1], 0, 0, 0);
                        oacc[4 * cc + 2] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a2, pt, oacc[4 * cc + 2], 0, 0, 0);
                        oacc[4 * cc + 3] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a3, pt, oacc[4 * cc + 3], 0, 0, 0);
                    }
                } else {
    #pragma unroll
                    for (int cc = 0; cc < D / 32; cc++) {
                        const uint32_t v0 = pb.v[0][cc], v1 = pb.v[1][cc], v2 = pb.v[2][cc], v3 = pb.v[3][cc];
                        const s16x4 ae = __builtin_bit_cast(s16x4, u32x2{__builtin_amdgcn_perm(v1, v0, 0x05040100u),
                                                                         __builtin_amdgcn_perm(v3, v2, 0x05040100u)});
                        const s16x4 ao = __builtin_bit_cast(s16x4, u32x2{__builtin_amdgcn_perm(v1, v0, 0x07060302u),
                                                                         __builtin_amdgcn_perm(v3, v2, 0x07060302u)});
                        oacc[2 * cc] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ae, pt, oacc[2 * cc], 0, 0, 0);
                        oacc[2 * cc + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ao, pt, oacc[2 * cc + 1], 0, 0, 0);
                    }
                }
            };

            // units of PU pages (two for FP8, whose pages are half the bytes, so
            // that as many bytes are in flight as for bf16): units j = wave,
            // wave + 4, ... with the next unit's loads in flight; the loads are
            // unconditional so that each wait covers exactly one unit (a page
            // past the chunk loads zeros and is masked)
            constexpr int PU = FP8 ? 2 : 1;
            struct Unit {
                PageBuf<D, FP8> p[PU];
            };
            auto load_u = [&](Unit& u, int j) {
    #pragma unroll
                for (int i = 0; i < PU; i++) load(u.p[i], PU * j + i);
            };
            auto compute_u = [&](const Unit& u, int j) {
    #pragma unroll
                for (int i = 0; i < PU; i++) compute(u.p[i], PU * j + i);
            };
            // publish this wavefront's state to LDS, then a workgroup barrier
            auto publish = [&](int set) {
                l_run = sum_xor32(sum_xor16(l_run));   // tokens of the four lane groups
                if (!exact) smax = max_xor32(max_xor16(smax));
                if (grp == 0) {
                    s_m[set][wave][col] = m_run;
                    s_l[set][wave][col] = l_run;
                    s_x[wave][col] = smax;
                }
                // Block i row 4grp + r -> dim 32(i/2) + 2(4grp + r) + i%2 (bf16),
                // 64(i/4) + 4(4grp + r) + i%4 (FP8; D = 128: 8(4grp + r) +
                // 4(i/4) + i%4), written 2 (bf16) or 4 (FP8) dims at a time.
                // Only the G real query rows (col < G) are read back; the 16
                // rows of a lane group lie D floats apart, in one LDS bank, so
                // writing the padding rows would only add bank conflicts.
                if (col < G) {
                    float* row = &s_o[set][wave][col][0];
                    if constexpr (FP8) {
    #pragma unroll
                        for (int w = 0; w < NB / 4; w++)
    #pragma unroll
                            for (int r = 0; r < 4; r++) {
                                const int d0 = D == 128 ? 8 * (4 * grp + r) + 4 * w : 64 * w + 4 * (4 * grp + r);
                                *(f32x4*)(row + d0) = f32x4{oacc[4 * w][r], oacc[4 * w + 1][r],
                                                            oacc[4 * w + 2][r], oacc[4 * w + 3][r]};
                            }
                    } else {
    #pragma unroll
                        for (int pp = 0; pp < NB / 2; pp++)
    #pragma unroll
                            for (int r = 0; r < 4; r++) {
                                typedef float f32x2 __attribute__((ext_vector_type(2)));
                                *(f32x2*)(row + 32 * pp + 2 * (4 * grp + r)) =
                                    f32x2{oacc[2 * pp][r], oacc[2 * pp + 1][r]};
                            }
                    }
                }
                __syncthreads();
            };
            const int nunits = (npg + PU - 1) / PU;
            const int nj = nunits > wave ? (nunits - wave + 3) / 4 : 0;
            Unit ba, bb;
            load_u(ba, wave);
            int n = 0;
            // every chunk but the last is full and gives every wavefront the
            // same, even number of units
            const int nb = a.split_tokens / (kPage * PU * 4);
            if constexpr (FP8) {
                // up to four chunks: each full chunk's state is published (the
                // two sets alternate) and merged while the next chunk's first
                // loads are in flight
                for (int h = 0; h + 1 < ncs; h++) {
                    for (; n < (h + 1) * nb; n += 2) {
                        load_u(bb, wave + 4 * (n + 1));
                        compute_u(ba, wave + 4 * n);
                        load_u(ba, wave + 4 * (n + 2));
                        compute_u(bb, wave + 4 * (n + 1));
                    }
                    publish(h & 1);
                    finish(c + h, h & 1);
                    m_run = exact ? -INFINITY : phi_l2;
                    l_run = 0.f;
                    smax = -INFINITY;
    #pragma unroll
                    for (int i = 0; i < NB; i++) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            } else if (ncs == 2) {
                // the first chunk's state is published to the first set while
                // the second chunk's first loads are in flight, and merged with
                // the second chunk's at the end of the item (merging it right
                // away measured 4% slower for bf16)
                for (; n < nb; n += 2) {
                    load_u(bb, wave + 4 * (n + 1));
                    compute_u(ba, wave + 4 * n);
                    load_u(ba, wave + 4 * (n + 2));
                    compute_u(bb, wave + 4 * (n + 1));
                }
                publish(0);
                m_run = exact ? -INFINITY : phi_l2;
                l_run = 0.f;
                smax = -INFINITY;
    #pragma unroll
                for (int i = 0; i < NB; i++) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            for (; n < nj; n += 2) {
                load_u(bb, wave + 4 * (n + 1));
                compute_u(ba, wave + 4 * n);
                if (n + 1 >= nj) break;
                load_u(ba, wave + 4 * (n + 2));
                compute_u(bb, wave + 4 * (n + 1));
            }
            publish(FP8 ? (ncs - 1) & 1 : (ncs == 2 ? 1 : 0));
        };

        if (a.unified) {
            pass(std::false_type{});
            // Rows (heads < G) whose largest scaled score leaves [phi - 60,
            // phi + 60] are recomputed with the exact pass: outside it a term
            // exp(s - phi) can overflow the fp32 sums (or the largest one
            // underflow).  Every thread reads the same LDS values, so the
            // decision is uniform across the workgroup.
            int n_out = 0;
            for (int g = 0; g < G; g++) {
                float M = -INFINITY;
                for (int w = 0; w < 4; w++) M = fmaxf(M, s_x[w][g]);
                // the raw scores are q.k of the cached values over k_scale
                // (1 for bf16): the scaled score is raw * scale * k_scale
                const float z = M * a.scale * a.k_scale - a.phi;
                if (z > kUnifiedWindow || z < -kUnifiedWindow) n_out++;
            }
            if (n_out > 0) {
                if (threadIdx.x == 0 && a.fallback_count) atomicAdd(a.fallback_count, n_out);
                __syncthreads();   // the LDS state is rewritten by the exact pass
                pass(std::true_type{});
            }
        } else {
            pass(std::true_type{});
        }

        if constexpr (FP8) finish(c + ncs - 1, (ncs - 1) & 1);
        else
            for (int h = 0; h < ncs; h++) finish(c + h, h);
        __syncthreads();   // the published states are rewritten by the next item
    };
    // persistent workgroups walk the (chunk, kv head, sequence) items; empty
    // chunks of short sequences cost a few scalar instructions
    const long n_items = (long)((a.max_splits - a.prefix_slots + cpi - 1) / cpi) * a.Hkv * a.B;
    for (long n = blockIdx.x; n < n_items; n += gridDim.x) {
        const int kvh = (int)(n % a.Hkv);
        const long r = n / a.Hkv;
        item((int)(r / a.B), kvh, (int)(r % a.B));
    }
}

}  // namespace

bool decode_mfma_supported(const DecodeArgs& a) {
    return !a.in_f32 && (a.D == 64 || a.D == 128) && a.Hq / a.Hkv <= kMaxG &&
           a.split_tokens <= 64 * kPage;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream) {
    const int cpi = chunks_per_item(a, a.in_fp8);
    const long n_items = (long)((a.max_splits - a.prefix_slots + cpi - 1) / cpi) * a.Hkv * a.B;
    // one item per workgroup up to 8192 items, then at most two (16384
    // workgroups at most): measured on the GQA workload's 32768 item slots,
    // 2 per workgroup ran 1.4-2.0% faster than 4, and 1 per workgroup slower
    const dim3 grid((unsigned)std::min<long>(
        n_items, std::min<long>(16384, std::max<long>(8192, (n_items + 1) / 2))));
    if (a.in_fp8) {
        if (a.D == 64) decode_mfma_kernel<64, true><<<grid, 256, 0, stream>>>(a);
        else decode_mfma_kernel<128, true><<<grid, 256, 0, stream>>>(a);
    } else {
        if (a.D == 64) decode_mfma_kernel<64, false><<<grid, 256, 0, stream>>>(a);
        else decode_mfma_kernel<128, false><<<grid, 256, 0, stream>>>(a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || (a.max_splits <= 1 && a.prefix_slots == 0)) return e;
    return launch_decode_combine(a, stream);
}

}  // namespace attn
