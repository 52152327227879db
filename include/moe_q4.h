/*
 * moe_q4.h - C ABI of the 4-bit grouped MoE layer for MI355X (gfx950).
 *
 * The layer: a router picks k of E experts per token and one shared expert
 * sees every token; each expert is a SwiGLU FFN whose weights are 4-bit
 * groupwise-affine codes (one bf16 scale and one bf16 bias per 64 weights).
 * Sources, by page and section:
 *   [P1] dothoosh.com, "Perplexity Lily: 1.35x faster decode for Qwen3.6 on
 *        Apple silicon": "Model specification" (256 experts, 8 selected plus
 *        a shared expert) and "Prefill optimizations" (fused dequantization
 *        in the grouped GEMM with FP32 accumulation; GPU-resident routing
 *        histogram, prefix scan, scatter and block map with no CPU sync;
 *        32-row tiles; bounded prefill chunks);
 *   [P3] droneth.or.th post on Lily: "A big model that touches only part of
 *        its weights per token" (format, bf16 expansion, ablations) and
 *        "Decode is limited by bandwidth more than by compute" (batch-1
 *        decode is bound by bytes moved).
 *
 * Conventions for every call below
 *   - All array pointers are DEVICE pointers owned by the caller, except the
 *     small argument structs themselves, which are HOST pointers read during
 *     the call only.  The caller keeps every buffer alive until the work
 *     enqueued on `stream` has finished.  Outputs must not alias inputs.
 *   - Every call only validates its arguments on the host and enqueues
 *     kernels on `stream`; it never allocates, frees or synchronises the
 *     host, and never reads device memory on the host.  Device-side values
 *     (such as n_blocks) stay on the device.
 *   - A call that fails its host-side checks returns a negative status and
 *     enqueues nothing.  No C++ exception crosses this boundary.  Device
 *     data (code words, scale values) is not validated.
 *   - Calls that enqueue more than one kernel (moe_route above its
 *     one-launch size, moe_grouped_gemm_q4, moe_layer_q4, moe_layer_chunked,
 *     moe_decode_q4 and its variants) check every argument before the first
 *     launch, but a launch itself can still fail (MOE_ERR_HIP, from
 *     hipGetLastError) after earlier kernels of the same call were enqueued.
 *     Those kernels then run; the call's outputs are undefined and the
 *     caller should treat the stream as failed.
 *   - The library holds no mutable global state except the scratch array of
 *     moe_decode_q4_noalloc (one per device, see there): other calls on
 *     different streams may run concurrently from different threads if their
 *     buffers differ.
 *   - Shapes: 1 <= k <= E <= 1000; H, I, I_sh are multiples of 64 (I_sh = 0
 *     means no shared expert); T >= 1; T*k*max(H, I) < 2^30 and
 *     T*max(H, I_sh) < 2^30 (bf16 byte offsets of x, h and the outputs fit
 *     in 31 bits); H*max(I, I_sh) < 2^32 (one expert's code words);
 *     block_rows is 16, 32 or 64.
 *   - Inputs are finite.  Scales must satisfy |s| < 2^118 (the kernels work
 *     with 512*s internally).
 *   - bf16 values travel as their uint16 bit patterns.
 */
#ifndef MOE_Q4_H
#define MOE_Q4_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MOE_OK                 0
#define MOE_ERR_NULL          -1  /* a required pointer is NULL */
#define MOE_ERR_SHAPE         -2  /* a size or block_rows outside the limits above */
#define MOE_ERR_ALIGN         -3  /* codes, x, y, expert_out or shared_out not 16-byte aligned,
                                     or a workspace not 256-byte aligned */
#define MOE_ERR_WORKSPACE     -4  /* workspace smaller than the matching *_workspace_bytes() */
#define MOE_ERR_HIP           -5  /* a kernel launch failed (hipGetLastError) */
#define MOE_ERR_UNIMPLEMENTED -6  /* combination not built into this library */

/* One set of 4-bit matrices [n_exp, N, K] (K innermost):
 *   codes  uint32, n_exp*N*K/8 words, 16-byte aligned: code of weight
 *          (n, 8c+i) in bits 4i..4i+3 of its word (lowest k in the low
 *          nibble); the words are ordered by `layout`:
 *            MOE_Q4_LAYOUT_ROWS   word (n, c) at n*(K/8) + c (row-major);
 *            MOE_Q4_LAYOUT_TILES  the tile-packed order moe_q4_prepack
 *                                 writes (see there);
 *            MOE_Q4_LAYOUT_TILES_SB  the same tile-packed order;
 *   scales bf16   [n_exp, N, K/64]: scale of weights (n, 64g .. 64g+63);
 *   biases bf16   [n_exp, N, K/64] (row-major in the first two layouts).
 *   MOE_Q4_LAYOUT_TILES_SB keeps each scale and its bias together in the
 *   order moe_q4_pack_scales writes: `scales` then points to n_exp*N*K/64
 *   uint32 words, word ((n/64)*(K/64) + g)*64 + n%64 holding the scale's
 *   bits in its low half and the bias's bits in its high half (n = e*N + n',
 *   4-byte aligned), and `biases` is not read (may be NULL).  The 64 rows of
 *   a tile then have their pairs for one group in 256 contiguous bytes, so a
 *   grouped-GEMM chunk reads them with its code words instead of keeping a
 *   table of the whole K in LDS.
 * Weight value: w = bf16_rne(fp32(q * scale + bias)) ([P1] "Prefill
 * optimizations"; [P3] "A big model ...").  Gate and up are [E, I, H],
 * down is [E, H, I]; the shared expert's are [1, I_sh, H] and [1, H, I_sh].
 * A zero-initialised layout is MOE_Q4_LAYOUT_ROWS.  The matrices passed to
 * one call must share one code-word order (ROWS, or TILES / TILES_SB); gate,
 * up, sh_gate and sh_up must share one layout; TILES_SB is accepted for the
 * gate and up matrices of every call (prefill and decode), not for down
 * matrices (MOE_ERR_SHAPE); moe_dequant_q4_bf16 expands row-major code words
 * only. */
#define MOE_Q4_LAYOUT_ROWS     0
#define MOE_Q4_LAYOUT_TILES    1
#define MOE_Q4_LAYOUT_TILES_SB 2
typedef struct {
    const uint32_t* codes;
    const uint16_t* scales;
    const uint16_t* biases;
    int32_t layout;
} moe_q4_mat;

/* Routing results of one layer call (all device arrays, caller-allocated).
 * Assignment a = t*k + j is token t's j-th expert.  [P1] "Prefill
 * optimizations" (histogram, prefix scan, scatter, block map); [P3] ablations.
 *   topk_idx      int32 [T, k]  experts by descending logit, ties -> lower index
 *   topk_w        fp32  [T, k]  softmax over the k selected logits
 *   counts        int32 [E]     assignments per expert (histogram)
 *   offsets       int32 [E+1]   exclusive prefix sum of counts; offsets[E] = T*k
 *   sorted_assign int32 [T*k]   row -> a, rows grouped by expert, ascending a inside one
 *   assign_row    int32 [T*k]   a -> row (inverse permutation)
 *   block_expert  int32 [max_blocks]  expert of row block b (-1 past n_blocks)
 *   block_row     int32 [max_blocks]  first row of block b (-1 past n_blocks)
 *   n_blocks      int32 [1]     number of blocks, written on the device
 * Block map: for e ascending, i < ceil(counts[e]/block_rows), block
 * (e, offsets[e] + block_rows*i) covering min(block_rows, counts[e] - block_rows*i) rows. */
typedef struct {
    int32_t* topk_idx;
    float*   topk_w;
    int32_t* counts;
    int32_t* offsets;
    int32_t* sorted_assign;
    int32_t* assign_row;
    int32_t* block_expert;
    int32_t* block_row;
    int32_t* n_blocks;
} moe_routing;

/* Version of this ABI (bumped on any change of a signature or of a call's
 * requirements, such as the workspace it needs; 4: moe_route takes a
 * workspace for k = 4, 8 or 16 above 64 tokens; 5: MOE_Q4_LAYOUT_TILES_SB
 * and moe_q4_pack_scales). */
int moe_abi_version(void);

/* Human-readable text of a status code (static string; never NULL). */
const char* moe_status_str(int status);

/* max_blocks = ceil(T*k / block_rows) + min(E, T*k): the length of
 * block_expert / block_row.  Returns a negative status on bad shapes. */
int moe_route_max_blocks(int T, int E, int k, int block_rows);

/* Device workspace bytes moe_route needs (0 on bad shapes).  With k = 4, 8 or
 * 16 and T above the one-launch size (T > 64, or a one-launch LDS need above
 * 64 KB) it is T*k 32-bit words, rounded up to 256 bytes: the top-k pass
 * records each 64-assignment chunk's match information there for the
 * grouping pass.  Otherwise it is 0 and ws may be NULL. */
size_t moe_route_workspace_bytes(int T, int E, int k, int block_rows);

/* GPU-resident routing ([P1] "Prefill optimizations", GPU-resident routing
 * bullet; [P1] "Model specification"; [P3] "A big model ...").
 *   logits  fp32 [T, E] router scores (device, 4-byte aligned, finite)
 *   out     host struct of device arrays described at moe_routing
 *   ws      device workspace of at least moe_route_workspace_bytes() bytes
 * Outputs are bit-exact functions of the logits (topk_w within fp32 rounding). */
int moe_route(const float* logits, int T, int E, int k, int block_rows,
              const moe_routing* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* Device workspace bytes moe_grouped_gemm_q4 needs (0 on bad shapes). */
size_t moe_gemm_workspace_bytes(int T, int H, int I, int I_sh, int E, int k, int block_rows);

/* Grouped expert GEMM with 4-bit dequantization fused into the tiles
 * ([P1] "Prefill optimizations", fused-dequantization bullet; [P3] "A big
 * model ...": weights expanded to bf16 tile by tile, FP32 accumulation,
 * expanded weights never written to memory).
 *   x          bf16 [T, H] activations (16-byte aligned)
 *   r          routing from moe_route with the same T, E, k, block_rows
 *   gate, up   [E, I, H] 4-bit matrices; down [E, H, I]
 *   sh_*       shared expert [1, I_sh, H] / [1, H, I_sh]; all NULL iff I_sh == 0
 *   expert_out bf16 [T*k, H]: row r = FFN of expert block_expert for token
 *              sorted_assign[r]/k, unweighted: (silu(x Wg^T) * (x Wu^T)) Wd^T
 *   shared_out bf16 [T, H]: shared expert FFN of every token (NULL iff I_sh == 0)
 *   ws         device workspace of at least moe_gemm_workspace_bytes() bytes
 * Accumulation is FP32; the SwiGLU activations and outputs are rounded to bf16. */
int moe_grouped_gemm_q4(const uint16_t* x, int T, int H, int I, int I_sh, int E, int k,
                        int block_rows, const moe_routing* r,
                        const moe_q4_mat* gate, const moe_q4_mat* up, const moe_q4_mat* down,
                        const moe_q4_mat* sh_gate, const moe_q4_mat* sh_up,
                        const moe_q4_mat* sh_down,
                        uint16_t* expert_out, uint16_t* shared_out,
                        void* ws, size_t ws_bytes, hipStream_t stream);

/* One whole layer call for T tokens: moe_route, moe_grouped_gemm_q4 and
 * moe_combine in one entry point, enqueued in that order on `stream`, with
 * the same arguments, buffers and results (routing r, expert_out,
 * shared_out and y are written exactly as by those three calls; [P1]
 * dothoosh.com "Prefill optimizations": GPU-resident routing feeding the
 * fused grouped GEMM with no CPU sync between them).
 *   route_ws: moe_route_workspace_bytes(T, E, k, block_rows) bytes (may be
 *             NULL when that is 0); gemm_ws: moe_gemm_workspace_bytes(...)
 *             bytes; both 256-byte aligned.  y bf16 [T, H], 16-byte aligned.
 * Status codes as for the three calls. */
int moe_layer_q4(const uint16_t* x, const float* logits, int T, int H, int I, int I_sh, int E,
                 int k, int block_rows, const moe_q4_mat* gate, const moe_q4_mat* up,
                 const moe_q4_mat* down, const moe_q4_mat* sh_gate, const moe_q4_mat* sh_up,
                 const moe_q4_mat* sh_down, const moe_routing* r, void* route_ws,
                 size_t route_ws_bytes, uint16_t* expert_out, uint16_t* shared_out,
                 void* gemm_ws, size_t gemm_ws_bytes, uint16_t* y, hipStream_t stream);

/* The two phases of moe_grouped_gemm_q4, for callers that schedule or time
 * them separately.  They share the workspace layout of moe_grouped_gemm_q4:
 * moe_expert_gateup_q4 writes the bf16 SwiGLU activations h (routed rows in
 * sorted-row order, then the shared expert's rows) into ws, and
 * moe_expert_down_q4 reads them from the same ws.  Calling both in order on
 * one stream equals moe_grouped_gemm_q4.
 *   gateup: h = bf16(silu(x Wg^T) * (x Wu^T)) per routed row and per token
 *           for the shared expert ([P1] "Prefill optimizations"; [P3]);
 *   down:   expert_out / shared_out = bf16(h Wd^T).
 * Arguments and status codes as for moe_grouped_gemm_q4; sh_gate/sh_up/sh_down
 * and shared_out are NULL iff I_sh == 0. */
int moe_expert_gateup_q4(const uint16_t* x, int T, int H, int I, int I_sh, int E, int k,
                         int block_rows, const moe_routing* r,
                         const moe_q4_mat* gate, const moe_q4_mat* up,
                         const moe_q4_mat* sh_gate, const moe_q4_mat* sh_up,
                         void* ws, size_t ws_bytes, hipStream_t stream);

int moe_expert_down_q4(int T, int H, int I, int I_sh, int E, int k, int block_rows,
                       const moe_routing* r, const moe_q4_mat* down, const moe_q4_mat* sh_down,
                       uint16_t* expert_out, uint16_t* shared_out,
                       const void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- Unfused baseline ([P2] aikraft.ru, "Technical optimizations: Prefill
 * and Decode"; [P3] droneth.or.th, ablation paragraph: the pages measure the
 * fused grouped GEMM against expanding the weights first). ---- */

/* Expand a 4-bit matrix set [n_exp, N, K] to bf16 [n_exp, N, K] (uint16 bit
 * patterns) in `out`, with the same arithmetic as the fused GEMM:
 * w = bf16_rne(fp32(q * scale + bias)).  counts: device int32 [n_exp] or
 * NULL; when given, experts with counts[e] == 0 are skipped and their rows of
 * `out` are left as they were.  out: n_exp*N*K*2 bytes, 16-byte aligned,
 * caller-owned.  K a multiple of 64, n_exp*N*K/8 < 2^31.  Enqueues one kernel. */
int moe_dequant_q4_bf16(const moe_q4_mat* m, int n_exp, int N, int K, const int32_t* counts,
                        uint16_t* out, hipStream_t stream);

/* moe_expert_gateup_q4 / moe_expert_down_q4 over weights already expanded to
 * bf16 (e.g. by moe_dequant_q4_bf16): gate/up bf16 [E, I, H], shared [1, I_sh, H],
 * down bf16 [E, H, I], shared [1, H, I_sh], each 16-byte aligned.  Same
 * routing, workspace and outputs as the 4-bit entry points; the GEMM tiles
 * and pipeline are the same, only the weight operand is read as bf16.
 * Shapes as for the 4-bit calls, and H*max(I, I_sh) < 2^30 (one expert's
 * bf16 matrix below 2^31 bytes). */
int moe_expert_gateup_bf16(const uint16_t* x, int T, int H, int I, int I_sh, int E, int k,
                           int block_rows, const moe_routing* r, const uint16_t* gate,
                           const uint16_t* up, const uint16_t* sh_gate, const uint16_t* sh_up,
                           void* ws, size_t ws_bytes, hipStream_t stream);

int moe_expert_down_bf16(int T, int H, int I, int I_sh, int E, int k, int block_rows,
                         const moe_routing* r, const uint16_t* down, const uint16_t* sh_down,
                         uint16_t* expert_out, uint16_t* shared_out, const void* ws,
                         size_t ws_bytes, hipStream_t stream);

/* Weighted combine: y[t] = sum_j topk_w[t,j] * expert_out[assign_row[t*k+j]]
 * + shared_out[t], summed in fp32 in slot order with the shared expert last
 * (weight 1; the pages name no shared-expert gate), rounded once to bf16.
 * shared_out may be NULL (no shared expert).  y bf16 [T, H], 16-byte aligned. */
int moe_combine(const uint16_t* expert_out, const uint16_t* shared_out, const moe_routing* r,
                int T, int H, int k, uint16_t* y, hipStream_t stream);

/* Weighted combine with a per-token weight on the shared expert:
 * y[t] = sum_j topk_w[t,j] * expert_out[assign_row[t*k+j]] + shared_gate[t] * shared_out[t],
 * fp32 sums in slot order, shared last, one bf16 rounding.  The pages name no
 * gate for the shared expert (moe_combine uses weight 1); this entry serves
 * models that gate it, e.g. with the gate output of moe_router.
 *   shared_gate: fp32 [T] device, 4-byte aligned; other arguments as moe_combine,
 *   except that shared_out is required. */
int moe_combine_gated(const uint16_t* expert_out, const uint16_t* shared_out,
                      const float* shared_gate, const moe_routing* r, int T, int H, int k,
                      uint16_t* y, hipStream_t stream);

/* Router projection ([P1] dothoosh.com, "Model specification": a router
 * scores the 256 experts of every token): the logits moe_route selects on.
 *   logits[t, e] = sum_h x[t, h] * w_router[e, h]  (bf16 in, fp32 accumulation)
 *   gate[t] = sigmoid(sum_h x[t, h] * w_gate[h])    (only when w_gate is given)
 * x bf16 [T, H], w_router bf16 [E, H], w_gate bf16 [H] (each 16-byte aligned);
 * logits fp32 [T, E] row-major, gate fp32 [T] (4-byte aligned), caller-owned.
 * w_gate and gate are both given or both NULL.  H a multiple of 64,
 * 1 <= E <= 1000.  Enqueues one kernel. */
int moe_router(const uint16_t* x, int T, int H, const uint16_t* w_router, int E,
               const uint16_t* w_gate, float* logits, float* gate, hipStream_t stream);

/* Repack the code words of a row-major matrix set [n_exp, N, K] into the
 * tile-packed order (load time; scales and biases keep their layout).  For
 * each expert, each tile of 64 rows and each run of 64 K, the 64 rows' 32
 * bytes are stored together: word (n, c) goes to
 *   e*N*K/8 + ((n'/64)*(K/64) + c/8)*512 + ((n'%64)/16)*128 + (n'%16)*8 + c%8
 * where n = e*N + n'.  A grouped-GEMM chunk of one tile is then one
 * contiguous 2 KB (64 K) or 4 KB (128 K) block instead of 64 row pieces,
 * which the memory system streams at a higher rate.  src and dst are
 * distinct device buffers of n_exp*N*K/8 words, 16-byte aligned; N and K
 * multiples of 64, n_exp*N*K/8 < 2^31.  Enqueues one kernel; the returned
 * matrix for later calls is {dst, src scales, src biases, MOE_Q4_LAYOUT_TILES}. */
int moe_q4_prepack(const uint32_t* src_codes, int n_exp, int N, int K, uint32_t* dst_codes,
                   hipStream_t stream);

/* Load time: the scales and biases of a matrix set [n_exp, N, K] (bf16
 * [n_exp, N, K/64] each, row-major) packed into the MOE_Q4_LAYOUT_TILES_SB
 * order: dst[((n/64)*(K/64) + g)*64 + n%64] = scale bits | bias bits << 16
 * for global row n = e*N + n' and group g.  dst: device, n_exp*N*K/64 words,
 * 4-byte aligned, distinct from the sources; N and K multiples of 64,
 * n_exp*N*K/64 < 2^31.  Enqueues one kernel; with moe_q4_prepack's codes the
 * matrix for later calls is {dst codes, dst, NULL, MOE_Q4_LAYOUT_TILES_SB}. */
int moe_q4_pack_scales(const uint16_t* scales, const uint16_t* biases, int n_exp, int N, int K,
                       uint32_t* dst, hipStream_t stream);

/* Streaming-read probe (measurement only): reads `bytes` of `buf` once with
 * 16-byte loads, one contiguous 32 KB range per workgroup, and writes the
 * XOR of range i's 32-bit words to sink[i] (a range past the end of buf is
 * shortened; its missing words count as zero).  Timing it over a buffer
 * larger than the 256 MB Infinity Cache gives the HBM read ceiling that the
 * weight-streaming kernels are compared against, next to the published
 * peak.
 *   buf: device, 16-byte aligned, bytes a positive multiple of 16
 *   sink: device, moe_read_probe_sink_words(bytes) uint32 words or more
 * Status: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN, MOE_ERR_WORKSPACE (sink
 * too short), MOE_ERR_HIP. */
size_t moe_read_probe_sink_words(size_t bytes);
int moe_read_probe(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words,
                   hipStream_t stream);

/* Launch-latency probe (measurement only): the floor under a chain of
 * dependent per-token launches such as moe_decode_q4's.  Enqueues n_launches
 * kernels on `stream`, alternating two shapes (grid_a workgroups of threads_a
 * threads, then grid_b of threads_b), the way a decode token's two launches
 * alternate.
 *   dep = 0: the kernels do nothing (launch and kernel-boundary cost only);
 *   dep = 1: launch i reads word i % 2 of buf in every workgroup and its
 *            workgroup 0 writes that value + 1 into word (i + 1) % 2, so each
 *            launch waits on the previous one's write through memory; from
 *            zeroed words, word n % 2 holds n after n launches.
 *   buf: device, 3 uint32 words, 4-byte aligned (word 2 is never written in
 *        practice: only when a read returns 0xFFFFFFFF).
 * Grids 1..65535, threads 64..1024 in multiples of 64, n_launches >= 1.
 * Status: MOE_ERR_NULL, MOE_ERR_ALIGN, MOE_ERR_SHAPE, MOE_ERR_HIP (a launch
 * failed after the earlier ones of the chain were enqueued). */
int moe_launch_probe(uint32_t* buf, int n_launches, int grid_a, int threads_a, int grid_b,
                     int threads_b, int dep, hipStream_t stream);

/* Device workspace bytes moe_decode_q4 needs (0 on bad shapes). */
size_t moe_decode_workspace_bytes(int H, int I, int I_sh, int E, int k);

/* Batch-1 decode of the whole layer for ONE token: two kernel launches on
 * `stream`, no host synchronisation ([P3] droneth.or.th, "Decode is limited
 * by bandwidth more than by compute"; [P1] dothoosh.com "Decode
 * optimizations", kernel-fusion bullet).
 * Computes the same function as moe_route + moe_grouped_gemm_q4 +
 * moe_combine at T = 1: top-k of the logits (identical selection and
 * weights), the k routed experts' and the shared expert's SwiGLU FFNs, and
 * the weighted sum, written to y.  Each weight-row dot is taken in the exact
 * affine form s * sum(q x) + b * sum(x) per 64-weight group in fp32, and the
 * per-expert outputs are summed in fp32 without the bf16 rounding of
 * expert_out, so y matches the three-call path up to rounding (h and y are
 * bf16, as there).  Deterministic: the same inputs give the same bits.
 *   x bf16 [1, H] (16-byte aligned), logits fp32 [1, E], y bf16 [1, H]
 *   r: routing arrays of this token (T = 1, block_rows as given), written
 *      exactly as moe_route would; may be NULL to skip them
 *   ws: at least moe_decode_workspace_bytes() bytes, 256-byte aligned;
 *      holds h and the chosen experts between the two launches
 * Limits: k <= 64. */
int moe_decode_q4(const uint16_t* x, const float* logits, int H, int I, int I_sh, int E, int k,
                  int block_rows, const moe_q4_mat* gate, const moe_q4_mat* up,
                  const moe_q4_mat* down, const moe_q4_mat* sh_gate, const moe_q4_mat* sh_up,
                  const moe_q4_mat* sh_down, const moe_routing* r, uint16_t* y, void* ws,
                  size_t ws_bytes, hipStream_t stream);

/* Largest workspace moe_decode_q4_noalloc can serve: the bytes of its
 * device-resident scratch array (256 KiB). */
size_t moe_decode_noalloc_max_bytes(void);

/* moe_decode_q4 without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The two launches, their results and the
 * status codes are those of moe_decode_q4; the workspace (h and the chosen
 * experts) is instead a file-scope device array of the library, one per GPU,
 * held until the process ends.  Its device address is looked up on the first
 * call on each device (hipGetSymbolAddress); no call allocates or frees.
 *   - Shapes whose moe_decode_workspace_bytes() exceeds
 *     moe_decode_noalloc_max_bytes() return MOE_ERR_WORKSPACE (with k = 8
 *     this allows max(I, I_sh) up to 14336).
 *   - Every call on one GPU uses the same array: calls that overlap on one
 *     GPU (different streams, or several host threads) race and give
 *     undefined results.  Calls in one stream's order are safe.  Nothing in
 *     the array needs to start at zero (each call writes what it reads).
 *   - MOE_ERR_HIP also when the device of `stream` cannot be queried or the
 *     array's address cannot be obtained. */
int moe_decode_q4_noalloc(const uint16_t* x, const float* logits, int H, int I, int I_sh, int E,
                          int k, int block_rows, const moe_q4_mat* gate, const moe_q4_mat* up,
                          const moe_q4_mat* down, const moe_q4_mat* sh_gate,
                          const moe_q4_mat* sh_up, const moe_q4_mat* sh_down,
                          const moe_routing* r, uint16_t* y, hipStream_t stream);

/* n_tok independent batch-1 decode calls, enqueued back to
 * back on `stream` (token t uses row t of x, logits and y; no batching across
 * tokens, no host synchronisation).  Same per-token result as moe_decode_q4
 * with r = NULL; the workspace is reused by each token in stream order. */
int moe_decode_q4_sequential(const uint16_t* x, const float* logits, int n_tok, int H, int I,
                             int I_sh, int E, int k, const moe_q4_mat* gate,
                             const moe_q4_mat* up, const moe_q4_mat* down,
                             const moe_q4_mat* sh_gate, const moe_q4_mat* sh_up,
                             const moe_q4_mat* sh_down, uint16_t* y, void* ws, size_t ws_bytes,
                             hipStream_t stream);

/* Device workspace bytes moe_layer_chunked needs for chunks of chunk_tokens. */
size_t moe_layer_workspace_bytes(int chunk_tokens, int H, int I, int I_sh, int E, int k,
                                 int block_rows);

/* Bounded-chunk driver ([P1] "Prefill optimizations", memory bullet: long
 * prompts run in bounded chunks so temporaries stay small).  Tokens
 * [c*chunk_tokens, ...) form independent layer calls (route, grouped GEMM,
 * combine) enqueued in order on `stream` with no host synchronisation.
 * All temporaries (routing, h, expert_out, shared_out) live in `ws` and are
 * sized for one chunk.  y bf16 [T, H].
 * Shapes: the size limits of the conventions above apply to one chunk
 * (C = min(chunk_tokens, T) tokens), since every kernel works inside one
 * chunk; the whole prompt needs only T*k < 2^30. */
int moe_layer_chunked(const uint16_t* x, const float* logits, int T, int H, int I, int I_sh,
                      int E, int k, int block_rows, int chunk_tokens,
                      const moe_q4_mat* gate, const moe_q4_mat* up, const moe_q4_mat* down,
                      const moe_q4_mat* sh_gate, const moe_q4_mat* sh_up,
                      const moe_q4_mat* sh_down,
                      uint16_t* y, void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_Q4_H */
