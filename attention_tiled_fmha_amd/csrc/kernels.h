// Host-side launchers of the gfx950 kernels.  Each launcher assumes its
// arguments were validated by the C ABI layer (attn_api.cpp) and returns the
// hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

// 1 in the checked build (libattn_checked.so): device-data checks with an
// error word, see common.h
#ifndef ATTN_CHECKED
#define ATTN_CHECKED 0
#endif

namespace attn {

// Compute units of the current device, read once per device; 256 (MI355X)
// when no device can be queried, so host-only planning calls still answer.
int device_cus();

// HBM read-rate probe: n_blocks blocks of hbm_probe_block_bytes() bytes, in
// `order` (or in place order when null).
int hbm_probe_block_bytes();
hipError_t launch_hbm_read(const void* buf, const int32_t* order, int n_blocks, uint32_t* sink,
                           hipStream_t stream);

// Dense prefill, bf16 in/out, bf16 MFMA with fp32 accumulation.
hipError_t launch_prefill_bf16(const void* q, const void* k, const void* v, void* o,
                               float* lse, int B, int Hq, int Hkv, int Tq, int Tk,
                               int D, bool causal, float scale, hipStream_t stream);

// Prefill of Tq new tokens per sequence against a paged bf16 cache
// [pages][Hkv][16][D]; sequence b has kv_lens[b] keys, its queries are its
// last Tq positions (causal diagonal at kv_lens[b] - Tq).
hipError_t launch_prefill_paged_bf16(const void* q, const void* k_pages, const void* v_pages,
                                     const int32_t* block_table, const int32_t* kv_lens,
                                     void* o, float* lse, int B, int Hq, int Hkv, int Tq, int D,
                                     int bt_stride, bool causal, float scale, hipStream_t stream,
                                     unsigned* err = nullptr, int num_pages = 0);

// Dense prefill, fp32 in/out, fp32 arithmetic (the exactness test mode).
hipError_t launch_prefill_f32(const float* q, const float* k, const float* v, float* o,
                              float* lse, int B, int Hq, int Hkv, int Tq, int Tk, int D,
                              bool causal, float scale, hipStream_t stream);

// Paged decode, split-KV.  One workgroup per (chunk, kv head, sequence).
// bt_stride is the row stride of the block table (0: every sequence reads
// row 0); kv_lens may be NULL, then every sequence has fixed_len tokens.
struct DecodeArgs {
    const void* q;
    const void* k_pages;
    const void* v_pages;
    const int32_t* block_table;
    long bt_stride;
    const int32_t* kv_lens;
    int fixed_len;
    int max_len;    // host bound; every length is clamped to [0, max_len]
    void* o;
    float* lse;
    float* ws_o;    // [B*Hq][max_splits][D] fp32 partial outputs
    float* ws_lse;  // [B*Hq][max_splits]    fp32 partial lse
    int B, Hq, Hkv, D;
    int split_tokens, max_splits;
    bool in_f32, out_f32;
    // FP8 cache (matrix-core kernel only): OCP E4M3 bytes, the cached value
    // being k_scale * e4m3 (keys) and v_scale * e4m3 (values); both scales
    // are 1 for bf16 / fp32 caches
    bool in_fp8;
    float k_scale, v_scale;
    float scale;
    // unified-max softmax (matrix-core kernel only): exponentials against phi,
    // exact recompute of the chunks whose rows leave the window; the number of
    // such (row, chunk) pairs is added to *fallback_count when it is not null
    bool unified;
    float phi;
    int* fallback_count;
    // cascade (matrix-core kernel only): workspace slots 0 .. prefix_slots - 1
    // of every row hold the prefix stage's chunk states; sequence chunk c goes
    // to slot prefix_slots + c (max_splits counts both, so no chunk is written
    // to the output directly) and the combine merges prefix_slots + nsplit(b)
    // slots of every row
    int prefix_slots;
    // checked build: the error word and the pool size the page indices are
    // checked against (unused otherwise)
    unsigned* err;
    int num_pages;
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// The same decode on the matrix core (bf16 or FP8 cache, G <= 16 query heads
// per kv head, chunks of at most 1024 tokens); decode_mfma_supported says
// whether launch_decode_mfma accepts the arguments.
bool decode_mfma_supported(const DecodeArgs& a);
hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream);

// Log-sum-exp combine of per-chunk partial states in the workspace into the
// output (rows = B*Hq, chunks = ceil(length / split_tokens)).
hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t stream);

// Shared-prefix stage of cascade decode (bf16 MFMA).  Work items are
// (prefix chunk of `chunk` tokens, kv head, block of 32 query rows), walked by
// a persistent grid; chunk is a multiple of 16 and at most 1024.  With more
// than one chunk the per-chunk states go to ws_o / ws_lse ([R*Hq][n_chunks][D],
// [R*Hq][n_chunks]) and must be combined with launch_decode_combine.
struct PrefixArgs {
    const void* q;           // [R, Hq, D] bf16
    const void* k_pages;     // [P, Hkv, 16, D] bf16 or E4M3 bytes
    const void* v_pages;
    const int32_t* pages;    // prefix pages
    int prefix_len;
    void* o;                 // [R, Hq, D] bf16 or fp32
    float* lse;              // [R, Hq] or null
    float* ws_o;
    float* ws_lse;
    int R, Hq, Hkv, D;
    int chunk;
    bool out_f32;
    // FP8 cache: E4M3 bytes, cached values k_scale * e4m3 and v_scale * e4m3
    // (both scales 1 for bf16)
    bool in_fp8;
    float k_scale, v_scale;
    float scale;
    // > 0: every chunk's state goes to workspace slot c of ws_slots per row
    // (the first slots of a cascade's decode workspace), also for one chunk
    int ws_slots;
    // checked build: error word and pool size (unused otherwise)
    unsigned* err;
    int num_pages;
};
hipError_t launch_prefix(const PrefixArgs& a, hipStream_t stream);

// In-place merge of two partial states.
hipError_t launch_merge_states(void* o_a, float* lse_a, const void* o_b, const float* lse_b,
                               int rows, int D, bool f32, hipStream_t stream);

// Flat GEMM C = A W^T (A [m][k], W [n][k] bf16; C [m][n] bf16 or fp32) for
// m <= 64.  A workgroup of `waves` wavefronts owns 16 * row_blocks rows of W
// (row_blocks 1, 2 or 4) and one of `splits` slices of steps_per_split 32-wide
// k steps; with splits > 1 the slices' fp32 partials go to ws
// ([splits][m][n]) and a second kernel adds them.  k is a multiple of 8.
struct FlatGemmArgs {
    const void* a;
    const void* w;
    void* c;
    float* ws;
    int m, n, k;
    int splits, steps_per_split;
    int row_blocks;
    int waves;          // wavefronts per workgroup: 4 or 8
    int lds_rows;       // > 0: the LDS-tiled kernel with this many rows of W per workgroup
    int chunks_per_split;   // LDS-tiled kernel: 64-wide k chunks per slice
    bool out_f32;
};
// k steps per register batch of the kernel instantiated for this m
int flat_gemm_batch_steps(int m, int row_blocks);
hipError_t launch_flat_gemm(const FlatGemmArgs& p, hipStream_t stream);

}  // namespace attn
