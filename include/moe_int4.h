/*
 * moe_int4.h -- C ABI of the MI355X (gfx950) int4 Mixture-of-Experts
 * feed-forward layer.
 *
 * The layer (discosf.com page "1 卡跑通 Llama 4", section "混合专家路由"):
 * a router scores every expert for each token, the top-k experts are chosen,
 * each chosen expert's SwiGLU FFN runs on its tokens and its output is added
 * back to the token weighted by the token's gate for that expert, and the
 * output of a shared expert that every token passes through is added last.
 * Expert FFN (docs.ifdog.com page "Llama 开源模型系列", section
 * "SwiGLU：门控激活的数学"): (Swish(x W1^T) * (x W3^T)) W2^T with
 * Swish(z) = z * sigmoid(z). Routed-expert weights are int4 in groups of 128
 * (same discosf.com page, section "FP8 / Int4 混合量化"), or of 64 or 32: the
 * smaller group sizes the lshu.cn page expects next (section "维护状态");
 * activations and the shared expert stay bf16 (lshu.cn page, section
 * "量化环节").
 *
 * Conventions for every entry point:
 *   - All data pointers are DEVICE pointers on the current HIP device, owned
 *     by the caller; the library never allocates or frees them and keeps no
 *     pointer after the call returns. `stream` is a hipStream_t (NULL = the
 *     default stream); work is enqueued asynchronously on it.
 *   - bf16 values are passed as uint16_t bit patterns.
 *   - Matrices are row-major. Weights are stored "nt": one row per output
 *     feature, the reduction dimension contiguous (W1, W3: [h, d]; W2: [d, h]).
 *   - Return value: MOE_OK, or an error code; nothing is enqueued when a
 *     validation error is returned. Faults during execution surface at the
 *     caller's next synchronisation. No C++ exception crosses the ABI.
 *     moe_last_error() gives a thread-local detail string for the last error.
 *   - Calls on one stream are ordered; concurrent calls on different streams
 *     must use distinct workspaces.
 */
#ifndef MOE_INT4_H
#define MOE_INT4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_INT4_ABI_VERSION 1

enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,        /* bad shape, null or misaligned pointer */
    MOE_ERR_UNSUPPORTED_DEVICE = 2, /* current device is not gfx950 */
    MOE_ERR_HIP = 3,                /* a HIP runtime call failed */
    MOE_ERR_WORKSPACE = 4           /* workspace missing or too small */
};

enum moe_path {
    MOE_PATH_AUTO = 0,     /* DECODE for at most 64 token-expert pairs; HYBRID when the
                              pairs average under 256 per routed expert; otherwise
                              PREFILL_WIDE */
    MOE_PATH_PREFILL = 1,  /* grouped GEMMs on MFMA for every expert, 128-row tiles */
    MOE_PATH_DECODE = 2,   /* HBM-streaming GEMV over the touched experts */
    MOE_PATH_HYBRID = 3,   /* grouped GEMMs for routed experts with more than 32 pairs
                              (128-row tiles) and for the shared expert (256-row tiles, a
                              launch of its own); routed experts with 1..32 pairs on the
                              streaming kernel, which reads their weights once instead of
                              padding them to GEMM tiles */
    MOE_PATH_PREFILL_WIDE = 4  /* PREFILL with 256 x 256 tiles (one block per CU, twice the
                              MFMA work per fragment read); pays off when experts hold
                              hundreds of rows */
};

/* Limits checked by validation. */
#define MOE_GROUP_SIZE 128     /* the default quantization group; 64 and 32 are also supported */
#define MOE_MAX_EXPERTS 256
#define MOE_MAX_TOP_K 16

/* Static description of an error code; never NULL. */
const char *moe_status_string(int status);

/* Detail text of the last error returned on the calling thread ("" if none). */
const char *moe_last_error(void);

/* MOE_INT4_ABI_VERSION of the built library. */
int moe_abi_version(void);

/* MOE_OK if the current HIP device is a gfx950, else MOE_ERR_UNSUPPORTED_DEVICE
 * (or MOE_ERR_HIP if there is no device). */
int moe_device_check(void);

/*
 * Int4 group quantizer (discosf.com page, section "FP8 / Int4 混合量化",
 * int4_row_quantize). For each group of `group_size` consecutive weights of a
 * row: scale = max(max|w|, 1e-6f) / 8, code = clamp(round_half_even(w / scale),
 * -8, 7), in fp32 with a correctly rounded division.
 *
 *   w       fp32 [rows, K], K % 128 == 0, 16-byte aligned
 *   q       out, uint8 [rows, K/2], 16-byte aligned: byte j of a row holds
 *           code 2j in its low nibble and code 2j+1 in its high nibble, 4-bit
 *           two's complement
 *   scales  out, fp32 [rows, K/group_size]
 *   group_size  128 (MOE_GROUP_SIZE), 64 or 32
 */
int moe_quantize_int4(const float *w, int64_t rows, int64_t K, int32_t group_size,
                      uint8_t *q, float *scales, void *stream);

/*
 * The same quantizer writing the tiled layout the forward pass reads
 * (MI355X-specific storage; codes and scales are bit-identical to
 * moe_quantize_int4, only their order in memory differs). rows % 16 == 0.
 * Tile (rb, g) covers rows 16*rb .. 16*rb+15 and reduction columns
 * 128*g .. 128*g+127; tiles are stored rb-major, t = rb * (K/128) + g. With
 * S = 128 / group_size scales per tile row:
 *   q       byte  t*1024 + ((k % 128)/32)*256 + (row % 16)*16 + (k % 32)/2
 *           (low nibble = even k)
 *   scales  float (t*16 + row % 16)*S + (k % 128)/group_size
 * A wavefront reads one 1 KB tile (and its 64*S B of scales) per access.
 */
int moe_quantize_int4_tiled(const float *w, int64_t rows, int64_t K, int32_t group_size,
                            uint8_t *q, float *scales, void *stream);

/*
 * Repack one matrix quantized by moe_quantize_int4 (the row-major format of
 * the quantizer on the discosf.com page, section "FP8 / Int4 混合量化") into
 * the tiled order moe_forward reads (the layout of moe_quantize_int4_tiled).
 * Bytes and scales move unchanged, so the result is bit-identical to
 * moe_quantize_int4_tiled on the same weights.
 *   q            uint8 [rows, K/2] row-major codes, 16-byte aligned
 *   scales       fp32 [rows, K/group_size] row-major scales
 *   rows         multiple of 16; K multiple of 128; group_size 128, 64 or 32
 *   q_tiled      out, rows*K/2 bytes, 16-byte aligned
 *   scales_tiled out, rows*K/group_size fp32
 * The row-major and tiled buffers must not overlap (MOE_ERR_INVALID_ARG).
 * Asynchronous on `stream`.
 */
int moe_tile_int4(const uint8_t *q, const float *scales, int64_t rows, int64_t K,
                  int32_t group_size, uint8_t *q_tiled, float *scales_tiled, void *stream);

/*
 * Repack a bf16 matrix [rows, K] (rows % 16 == 0, K % 128 == 0) into the
 * tiled order the forward pass reads for the shared expert: tile
 * t = (row/16) * (K/128) + k/128 holds 16 rows x 128 columns as 4 steps of
 * 32 columns, element (row, k) at
 *   t*2048 + ((k % 128)/32)*512 + (row % 16)*32 + (k % 32).
 * src and dst are device buffers of rows*K bf16 and must not overlap.
 */
int moe_pack_bf16_tiled(const uint16_t *src, int64_t rows, int64_t K, uint16_t *dst,
                        void *stream);

typedef struct moe_dims {
    int64_t T;      /* tokens, >= 1 */
    int64_t d;      /* model dim, multiple of 128 */
    int64_t E;      /* routed experts, 1..MOE_MAX_EXPERTS */
    int64_t h;      /* expert hidden dim, multiple of 128 */
    int32_t top_k;  /* 1..min(E, MOE_MAX_TOP_K) */
    int32_t group_size; /* int4 quantization group: 128, 64 or 32 */
} moe_dims;

/* Routed experts, each matrix in the TILED int4 layout: written by
 * moe_quantize_int4_tiled with dims->group_size (g), or by moe_quantize_int4
 * and then moe_tile_int4. Row-major codes passed here are read as tiles and
 * give wrong results (the layouts cannot be told apart from the bytes).
 * Experts are stacked (expert e's matrix starts at e times the matrix size):
 *   w1q, w3q [E] x tiled [h, d]: E*h*d/2 bytes   w1s, w3s: E*h*d/g fp32
 *   w2q      [E] x tiled [d, h]: E*d*h/2 bytes   w2s:      E*d*h/g fp32 */
typedef struct moe_experts_int4 {
    const uint8_t *w1q, *w3q, *w2q;
    const float *w1s, *w3s, *w2s;
} moe_experts_int4;

/* Shared expert, bf16, each matrix packed by moe_pack_bf16_tiled:
 * s1, s3 from [h, d]; s2 from [d, h]. */
typedef struct moe_shared_bf16 {
    const uint16_t *s1, *s3, *s2;
} moe_shared_bf16;

/* Bytes of device workspace moe_forward / moe_route need for `dims`
 * (0 if dims are invalid). */
size_t moe_forward_workspace_bytes(const moe_dims *dims);

/*
 * The MoE feed-forward layer.
 *   x          bf16 [T, d]
 *   router_w   fp32 [E, d]; logit[t,e] = sum_j x[t,j] router_w[e,j] (+ router_b[e])
 *   router_b   fp32 [E] or NULL
 *   experts    routed int4 experts (see moe_experts_int4)
 *   shared     shared bf16 expert
 *   y          out, bf16 [T, d]:
 *              y[t] = shared(x_t) + sum_j gate[t,j] * expert_{id[t,j]}(x_t)
 *   topk_ids   out, int32 [T, top_k] or NULL: chosen experts by descending
 *              logit, ties to the lower id
 *   topk_gates out, fp32 [T, top_k] or NULL: sigmoid of the chosen logits
 *   workspace  device buffer of >= moe_forward_workspace_bytes(dims) bytes,
 *              256-byte aligned; contents are scratch
 * Accumulation is fp32; the only roundings beyond fp32 are the bf16 inputs of
 * the matrix cores (dequantized weights, SwiGLU hidden rows) and the bf16 y.
 */
int moe_forward(const moe_dims *dims, const uint16_t *x, const float *router_w,
                const float *router_b, const moe_experts_int4 *experts,
                const moe_shared_bf16 *shared, uint16_t *y, int32_t *topk_ids,
                float *topk_gates, void *workspace, size_t workspace_bytes,
                void *stream);

/* moe_forward with an explicit path (enum moe_path). */
int moe_forward_path(const moe_dims *dims, const uint16_t *x, const float *router_w,
                     const float *router_b, const moe_experts_int4 *experts,
                     const moe_shared_bf16 *shared, uint16_t *y, int32_t *topk_ids,
                     float *topk_gates, int32_t path, void *workspace,
                     size_t workspace_bytes, void *stream);

/*
 * moe_forward_path without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. The workspace is a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES inside the library (each GPU the library runs on
 * holds its own copy until the process ends); nothing is allocated or freed by
 * a call. Layers whose moe_forward_workspace_bytes(dims) exceed it return
 * MOE_ERR_WORKSPACE (64 MiB holds, e.g., up to about 550 tokens at top-1 with
 * d = 5120, h = 8192).
 * The first call on a device does a one-time set-up there (the array's device
 * address and the library's second stream for the hybrid path); make it
 * outside graph capture. Every call on a GPU shares that GPU's array and
 * leaves its contents behind: calls that overlap on one GPU (different
 * streams, or host threads) race on it and must be serialised by the caller.
 * Stage timing (moe_profile_enable) creates events; keep it off here.
 * Arguments, outputs, paths and errors otherwise as moe_forward_path.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_forward_noalloc(const moe_dims *dims, const uint16_t *x, const float *router_w,
                        const float *router_b, const moe_experts_int4 *experts,
                        const moe_shared_bf16 *shared, uint16_t *y, int32_t *topk_ids,
                        float *topk_gates, int32_t path, void *stream);

/* Row-wise fp8 (OCP E4M3) quantization of the fp8 routed-expert path: the
 * lshu.cn page (section "量化环节") quantizes each activation row to fp8 with
 * its scale bounded by activation_scale_ub, and holds the weights in fp8 with
 * one scale per row ("FP8 行级", section "三条推理路径差异"). Per row of K
 * values, in fp32 with a correctly rounded division:
 *   scale = min(max(max|v|, 1e-12), ub) / 448,   code = fp8_rne(clamp(v / scale, -448, 448))
 * (no bound for weights; ub <= 0: no bound).
 *
 * moe_quantize_fp8_tiled: weights, w fp32 [rows, K] row-major, rows % 16 == 0,
 *   K % 128 == 0 -> q [rows * K] bytes in the tiled order the forward reads
 *   (tile t = (row/16)*(K/128) + k/128 of 2 KB; byte
 *   t*2048 + ((k%128)/32)*512 + (row%16)*32 + k%32), scales fp32 [rows].
 *   w 16-byte aligned; q and scales 4-byte aligned.
 * moe_quantize_fp8_rows: activations, x bf16 [rows, K] row-major -> q [rows, K]
 *   row-major codes, scales fp32 [rows]. x 8-byte aligned.
 * Both: INVALID_ARG on bad shapes / pointers; asynchronous on `stream`. */
int moe_quantize_fp8_tiled(const float *w, int64_t rows, int64_t K, uint8_t *q, float *scales,
                           void *stream);
int moe_quantize_fp8_rows(const uint16_t *x, int64_t rows, int64_t K, float ub, uint8_t *q,
                          float *scales, void *stream);

/* Routed experts in bf16: the pure-bf16 inference path, which the lshu.cn
 * page "Llama 4 单卡量化推理与选型指南" (section "三条推理路径差异") lists as
 * the accuracy baseline of the int4 and fp8 paths. Each expert's matrix is
 * packed by moe_pack_bf16_tiled and the experts are stacked:
 *   w1, w3 [E] x tiled [h, d]: E*h*d bf16     w2 [E] x tiled [d, h]: E*d*h bf16 */
typedef struct moe_experts_bf16 {
    const uint16_t *w1, *w3, *w2;
} moe_experts_bf16;

/* moe_forward_path with bf16 routed experts: the same layer, workspace, paths,
 * outputs and errors; the routed FFNs use the bf16 weights as given. */
int moe_forward_bf16(const moe_dims *dims, const uint16_t *x, const float *router_w,
                     const float *router_b, const moe_experts_bf16 *experts,
                     const moe_shared_bf16 *shared, uint16_t *y, int32_t *topk_ids,
                     float *topk_gates, int32_t path, void *workspace,
                     size_t workspace_bytes, void *stream);

/* Routed experts in fp8 (OCP E4M3) with one fp32 scale per weight row: the
 * fp8_mixed path of the lshu.cn page "Llama 4 单卡量化推理与选型指南"
 * (sections "三条推理路径差异" and "量化环节"). Each matrix is written by
 * moe_quantize_fp8_tiled and the experts are stacked:
 *   w1q, w3q [E] x tiled [h, d]: E*h*d bytes   w1s, w3s: E*h fp32
 *   w2q      [E] x tiled [d, h]: E*d*h bytes   w2s:      E*d fp32
 * act_ub: the activation scale upper bound (finite, >= 0; 0: no bound). */
typedef struct moe_experts_fp8 {
    const uint8_t *w1q, *w3q, *w2q;
    const float *w1s, *w3s, *w2s;
    float act_ub;
} moe_experts_fp8;

/* Bytes of device workspace moe_forward_fp8 needs for `dims` (0 if invalid):
 * the moe_forward workspace plus the fp8 activation rows and their scales. */
size_t moe_forward_fp8_workspace_bytes(const moe_dims *dims);

/* moe_forward_path with fp8 routed experts. Each routed expert computes, as
 * on the page: x_t quantized per row (moe_quantize_fp8_rows with act_ub);
 * a1 = bf16(xq W1q^T * sx * s1), a3 = bf16(xq W3q^T * sx * s3) (exact fp8
 * products, fp32 sums); h = bf16(silu(a1) a3); h quantized per row the same
 * way; out = bf16(hq W2q^T * sh * s2). The router, the shared bf16 expert,
 * the gates, combine, paths, outputs and errors are those of moe_forward_path;
 * workspace >= moe_forward_fp8_workspace_bytes(dims). */
int moe_forward_fp8(const moe_dims *dims, const uint16_t *x, const float *router_w,
                    const float *router_b, const moe_experts_fp8 *experts,
                    const moe_shared_bf16 *shared, uint16_t *y, int32_t *topk_ids,
                    float *topk_gates, int32_t path, void *workspace,
                    size_t workspace_bytes, void *stream);

/* Bytes of device workspace moe_route alone needs (a prefix of the forward
 * workspace; 0 if dims are invalid; dims->h is ignored). */
size_t moe_route_workspace_bytes(const moe_dims *dims);

/*
 * Routing alone: router logits, top-k + sigmoid gates, and the token->expert
 * dispatch the grouped GEMMs use (discosf.com page, section "混合专家路由").
 * Pairs are p = t * top_k + j. Every output except topk_ids/topk_gates may be
 * NULL.
 *   logits   out, fp32 [T, E] (bias included)
 *   counts   out, int32 [E]: pairs routed to each expert
 *   offsets  out, int32 [E+1]: exclusive prefix sum of counts
 *   perm     out, int32 [T*top_k]: perm[slot] = pair; slots of expert e are
 *            offsets[e]..offsets[e+1]-1, pairs in ascending order
 *   inv      out, int32 [T*top_k]: inv[pair] = slot
 *   workspace >= moe_route_workspace_bytes(dims) bytes, 256-byte aligned
 */
int moe_route(const moe_dims *dims, const uint16_t *x, const float *router_w,
              const float *router_b, int32_t *topk_ids, float *topk_gates,
              float *logits, int32_t *counts, int32_t *offsets, int32_t *perm,
              int32_t *inv, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Per-stage timing for benchmarks (not part of the layer's arithmetic).
 * While enabled, each stage of every moe_forward / moe_route call (and each
 * int4 quantizer call, as MOE_STAGE_QUANTIZE) is timed by
 * a pair of hipEvents that its kernels record themselves (hipExtLaunchKernel):
 * at the start of the stage's first kernel and the end of its last, so the
 * time excludes the dispatch gap before the stage. moe_profile_read waits for
 * the recorded events, writes the summed duration in milliseconds and the
 * number of timed stage calls of each stage (arrays of `n` entries,
 * n <= MOE_STAGE_COUNT), and resets the sums. It is off by default; while off,
 * kernels launch plainly (and can be captured in graphs). State is
 * process-wide; it is not meant for concurrent callers.
 */
enum moe_stage {
    MOE_STAGE_ROUTER = 0,      /* K2 router logits */
    MOE_STAGE_TOPK = 1,        /* K2 top-k + gates */
    MOE_STAGE_DISPATCH = 2,    /* K3 */
    MOE_STAGE_UP = 3,          /* K4 + shared up-projection, SwiGLU */
    MOE_STAGE_DOWN = 4,        /* K5 + shared down-projection */
    MOE_STAGE_COMBINE = 5,     /* gate-weighted sum + shared, bf16 out */
    MOE_STAGE_DECODE_UP = 6,   /* decode path: streaming up-projection */
    MOE_STAGE_DECODE_DOWN = 7, /* decode path: streaming down-projection */
    MOE_STAGE_ACT_QUANT = 8,   /* fp8 experts: per-row fp8 quantization of x and H */
    MOE_STAGE_QUANTIZE = 9,    /* K1: moe_quantize_int4 / moe_quantize_int4_tiled calls */
    MOE_STAGE_COUNT = 10
};

/*
 * HBM measurement helpers for benchmarks (not part of the layer's arithmetic):
 * the rates plain streaming reaches on the device, the practical ceiling beside
 * the nominal peak. Device pointers, asynchronous on `stream`; bytes must be a
 * positive multiple of 16 and the pointers 16-byte aligned (MOE_ERR_INVALID_ARG
 * otherwise).
 *   moe_hbm_read: reads every 16-byte word of buf once with the non-temporal
 *     loads of the streaming decode kernels; block b of the launch writes the
 *     XOR of the 32-bit words it read to sink[b] (sink: moe_hbm_read_sink_words()
 *     uint32 words, caller-owned), so the XOR of all sink words is the XOR of
 *     the buffer's words.
 *   moe_hbm_copy: copies bytes from src to dst (buffers must not overlap).
 */
int moe_hbm_read(const void *buf, int64_t bytes, uint32_t *sink, void *stream);
int moe_hbm_read_sink_words(void);
int moe_hbm_copy(void *dst, const void *src, int64_t bytes, void *stream);

int moe_profile_enable(int on);
int moe_profile_read(double *ms, int64_t *launches, int n);
const char *moe_stage_name(int stage);

#ifdef __cplusplus
}
#endif

#endif /* MOE_INT4_H */
