/*
 * q4.h -- C ABI of libq4stream, the MI355X (gfx950) INT4 weight-streaming
 * decode library.
 *
 * The library computes the per-token matrix-vector product over 4-bit,
 * group-quantized weights without writing dequantized weights to memory
 * (PIPO: Pipelined Offloading for Efficient Inference on Consumer Devices,
 * "Method", bullet "Computation optimization"), a small-batch variant of it
 * for batches below 16 (same page, bullet "Automatic configuration", and
 * "Limitations"), a per-token layer loop captured once per context-length
 * bucket as a HIP graph (PipeLLM: Faster Local LLM Inference Than llama.cpp
 * via System-Level Optimizations, "Layer 1: CUDA Graph Compilation"), and
 * double-buffered streaming of whole layers from pinned host memory over a
 * copy stream (same page, "Layer 2: Asynchronous Weight Prefetching"; PIPO,
 * "Method", bullets "Pipeline design", "Two pipeline modes" and "Data
 * transfer suite").
 *
 * Weight format (the pages give no bit layout; this is the reading used):
 *   - N x K matrix, K a multiple of 32;
 *   - packed: u8[N][K/2], row-major; byte j of row n holds the unsigned code
 *     of column 2j in bits 0..3 and of column 2j+1 in bits 4..7;
 *   - scales: IEEE binary16 bit patterns u16[N][K/32], row-major, one per
 *     group of 32 consecutive columns;
 *   - weight w[n][k] = scale[n][k/32] * (code[n][k] - 8).
 * Activations are binary16 bit patterns; outputs and the residual are fp32.
 *
 * Conventions for every function below:
 *   - Pointers are DEVICE pointers unless marked "host".  The library never
 *     allocates, frees or retains caller memory beyond the objects
 *     documented as retaining pointers (decoder, weight stream).
 *   - GPU work is enqueued on the given stream and is asynchronous with
 *     respect to the host; a NULL stream means the default stream.
 *   - Arguments are validated on the host before anything is enqueued; on
 *     error nothing is enqueued and a non-zero status is returned, with a
 *     message available from q4_last_error() on the same thread.
 *   - Faults inside a kernel surface at the caller's next synchronisation.
 *   - Every kernel uses a fixed reduction order and no floating-point
 *     atomics: repeated calls give bitwise identical results.
 *   - Distinct objects may be used from distinct threads; one object must
 *     not be used from two threads at once.
 */
#ifndef Q4_H
#define Q4_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q4_ABI_VERSION 5

typedef int32_t q4_status;
#define Q4_OK 0
#define Q4_ERR_INVALID_ARG 1 /* bad pointer, size, alignment or range */
#define Q4_ERR_UNSUPPORTED 2 /* valid request outside what is implemented */
#define Q4_ERR_HIP 3         /* a HIP runtime call failed */
#define Q4_ERR_STATE 4       /* call out of order (e.g. wait before begin) */
#define Q4_ERR_OOM 5         /* host allocation failed */

/* Largest K accepted by the products (the activation vector of one
 * workgroup lives in LDS: 2*K bytes). */
#define Q4_MAX_K 32768
/* Largest batch of q4_gemm_smallbatch. */
#define Q4_MAX_BATCH 16

/* Message for the last non-OK status returned on this thread ("" if none).
 * The string stays valid until the next library call on this thread. */
const char *q4_last_error(void);
int32_t q4_abi_version(void);

/* ------------------------------------------------------------------ */
/* Packing                                                              */
/* ------------------------------------------------------------------ */

/* Packing of 4-bit codes (PIPO, "Method", bullet "Computation
 * optimization": the product runs on 4-bit quantized weights; the pages fix
 * no byte layout, so the layout is the reading stated at the top of this
 * file: two codes per byte, the even column in the low nibble).
 * codes u8[N][K] (one code per byte; only bits 0..3 are used, higher bits
 * are ignored) -> packed u8[N][K/2] in the layout above.  N >= 1, K >= 2
 * and even.  Bit-exact; no alignment requirement. */
q4_status q4_pack(const uint8_t *codes, uint8_t *packed, int64_t N, int64_t K,
                  hipStream_t stream);

/* The inverse of q4_pack (same passage and layout): packed u8[N][K/2] ->
 * codes u8[N][K] (each 0..15).  Same limits and errors as q4_pack. */
q4_status q4_unpack(const uint8_t *packed, uint8_t *codes, int64_t N,
                    int64_t K, hipStream_t stream);

/* ------------------------------------------------------------------ */
/* Quantization of real weights                                         */
/* ------------------------------------------------------------------ */

#define Q4_DTYPE_F32 0
#define Q4_DTYPE_F16 1

/* Real weights -> the 4-bit format above (PIPO, "Method", "Computation
 * optimization" runs on 4-bit weights but gives no rule to produce them;
 * the rule here is symmetric round-to-nearest per group of 32 k):
 *   s = binary16(max|w| / 8) over the group (nearest even);
 *   code = clamp(rint(w / s) + 8, 0, 15), w / s the exact quotient (one
 *   IEEE binary32 division decides its rounding exactly for binary32 or
 *   binary16 w and binary16 s), rint ties to even; a group whose s is 0
 *   gets code 8 everywhere.
 * The largest positive weight of a group maps to w / s = 8, clipped to 15.
 *   w       device [N][K], row-major, w_dtype Q4_DTYPE_F32 (binary32) or
 *           Q4_DTYPE_F16 (binary16 bit patterns), 16-byte aligned; finite,
 *           with max|w| / 8 < 65520 per group (else the scale is infinite);
 *   packed  device u8[N][K/2] out, 16-byte aligned;
 *   scales  device u16[N][K/32] out, 2-byte aligned.
 * N >= 1, K >= 32, K % 32 == 0; INVALID_ARG otherwise, nothing enqueued.
 * Bit-exact: the same codes and scales on every run. */
q4_status q4_quantize(const void *w, int32_t w_dtype, uint8_t *packed,
                      uint16_t *scales, int64_t N, int64_t K, hipStream_t stream);

/* ------------------------------------------------------------------ */
/* Products (PIPO, "Method", "Computation optimization")                 */
/* ------------------------------------------------------------------ */

/* y[n] = sum_k w[n][k] * x[k] for n < N.
 *   packed  u8[N][K/2], 16-byte aligned;  scales u16[N][K/32], 2-byte aligned;
 *   x_f16   u16[K] binary16, 16-byte aligned;  y f32[N], 4-byte aligned.
 *   1 <= N <= 2^31-1;  32 <= K <= Q4_MAX_K;  K % 32 == 0.
 * Each group's 32 products are formed exactly (binary16 x binary16) and
 * summed in fp32, then scaled by the group's scale in fp32. */
q4_status q4_gemv(const uint8_t *packed, const uint16_t *scales,
                  const uint16_t *x_f16, float *y, int64_t N, int64_t K,
                  hipStream_t stream);

/* Y[b][n] = sum_k w[n][k] * X[b][k] for b < B, n < N.
 *   X_f16 u16[B][K] binary16 (each activation vector contiguous),
 *   16-byte aligned;  Y f32[B][N], 4-byte aligned;  1 <= B <= Q4_MAX_BATCH;
 *   other arguments as q4_gemv.  B == 1 runs the q4_gemv kernel; 2 <= B <= 3
 *   with B * K * 2 <= 65536 runs the vector-ALU batch kernel, whose every
 *   column equals q4_gemv of that column bitwise; wider batches run the
 *   matrix-core kernel, whose columns do not depend on B or on the other
 *   columns (bitwise), and differ from q4_gemv within the product bound.
 *   Every path forms each group's 32 products exactly (the codes as the
 *   integers -8..7 against binary16 activations), sums them in fp32 and
 *   scales the sum by the group's scale in fp32, so every finite binary16
 *   scale, subnormal ones included, is honoured. */
q4_status q4_gemm_smallbatch(const uint8_t *packed, const uint16_t *scales,
                             const uint16_t *X_f16, float *Y, int64_t N,
                             int64_t K, int32_t B, hipStream_t stream);

/* ------------------------------------------------------------------ */
/* Decode step (PipeLLM, "Layer 1: CUDA Graph Compilation")               */
/* ------------------------------------------------------------------ */

typedef struct {
    const uint8_t *packed;  /* device u8[N][K/2], 16-byte aligned */
    const uint16_t *scales; /* device u16[N][K/32] */
    int64_t N, K;
} q4_matrix;

/* One decoder layer: fused QKV (rows Q | K | V), O, fused gate+up
 * (rows gate | up) and down. */
typedef struct {
    q4_matrix qkv, o, gate_up, down;
} q4_layer;

typedef struct {
    int32_t n_layers;
    int32_t d_model;    /* d */
    int32_t n_heads;    /* H query heads */
    int32_t n_kv_heads; /* Hkv key/value heads, H % Hkv == 0 */
    int32_t head_dim;   /* hd */
    int32_t d_ff;       /* dff */
    float eps;          /* RMSNorm epsilon */
    /* host array of n_layers layers, copied at create; may be NULL when the
     * decoder is only driven layer by layer (q4_decode_layer). */
    const q4_layer *layers;
    float *h;                  /* device f32[d], 16-byte aligned: residual in/out, retained */
    /* device, 256-byte aligned, retained.  After a layer it holds, each
     * section starting at a 256-byte boundary in this order: the binary16
     * normed input of gate+up, i.e. the second norm (max(d, dff) slots), the fp32
     * QKV output ((H + 2*Hkv)*hd), the binary16 attention output (H*hd),
     * the binary16 gated MLP activation (dff), 256 bytes of barrier words
     * and the device layer table (n_layers entries of 64 bytes). */
    void *workspace;
    size_t workspace_bytes;    /* >= q4_decoder_workspace_bytes() */
    /* Attention over a KV cache, optional (PipeLLM, "Layer 1: CUDA Graph
     * Compilation": graphs per sequence-length bucket; PIPO, "Method",
     * "Pipeline design": KV cache state beside the weights).  NULL: the
     * one-token stand-in described below.  Otherwise device binary16 caches,
     * 16-byte aligned, retained, 2 * n_layers * n_kv_heads * max_ctx *
     * head_dim elements: for layer l the keys at element offset
     * 2*l*S and the values at (2*l + 1)*S, S = n_kv_heads*max_ctx*head_dim,
     * each laid out [n_kv_heads][max_ctx][head_dim].  A step at context
     * length c stores the current token's rotated key and its value in row
     * c - 1 and attends over rows 0..c-1.  With a cache the workspace also
     * holds, after the layer table, a position word (256 bytes), the
     * per-chunk attention partials, the rotated queries (n_heads * head_dim *
     * 4 bytes per column) and a rotation table (max_ctx * head_dim * 4
     * bytes), each 256-byte aligned.  Needs n_heads / n_kv_heads in {1, 2, 4, 8} and head_dim
     * 64 or 128; only the four-kernels step (mode 0). */
    void *kv_cache;
    int32_t max_ctx;           /* rows per cache, 1..2^20 */
    float rope_base;           /* rotary base (theta), > 0, e.g. 500000 */
    /* Batched verify step (PipeInfer, "Run" / "Tuning PipeInfer":
     * speculative micro-batches of a few draft tokens; PIPO, "Method",
     * "Automatic configuration": 4-bit kernel below batch 16).  max_batch
     * 0 = none, else 1..16 columns; h_batch: device f32[max_batch][d_model],
     * 16-byte aligned, retained, the residual columns in/out.  With
     * max_batch > 0 the workspace also holds, after the sections above,
     * 256-byte aligned: binary16 [max_batch][d_model] (normed input),
     * fp32 [max_batch][(H + 2 Hkv) hd] (QKV), binary16 [max_batch][H hd]
     * (attention output), binary16 [max_batch][d_ff] (gated MLP
     * activation).  With a KV cache too, the
     * attention partials and rotated queries are sized for max_batch
     * columns. */
    int32_t max_batch;
    float *h_batch;
} q4_model_desc;

/*
 * Per layer, on the fp32 residual h (a reading: the pages list the four
 * products of a decode layer but none of the glue between them):
 *   a   = f16(h / sqrt(mean(h^2) + eps))
 *   qkv = Wqkv a;  o = f16(V of the key/value group of each query head)
 *   h  += Wo o
 *   a2  = f16(h / sqrt(mean(h^2) + eps))
 *   gu  = Wgu a2;  m = f16(silu(gate) * up)
 *   h  += Wdown m
 * The gather is one-token attention: with a single cached key, softmax is 1
 * and rotary position 0 is the identity.
 */
q4_status q4_decoder_workspace_bytes(const q4_model_desc *m, size_t *out);
/* Validates and copies the description.  Shapes must match the dimensions
 * and satisfy the q4_gemv limits.  With resident layers it also writes, with
 * synchronous copies, a device copy of the layer table and zeroed barrier
 * words into the workspace; the step starts as four kernels per layer (the
 * persistent step below is opt-in).  With a KV cache it zeroes the position
 * word (context length 1) and fills the rotation table (cos and sin of every
 * position's angles, taken in fp64), synchronously.  Otherwise no GPU work. */
q4_status q4_decoder_create(const q4_model_desc *m, void **dec);
/* Step implementation for resident layers (cached graphs are dropped on a
 * change):
 *   0 four kernels per layer (the default);
 *   1 one persistent kernel per token: all layers, products separated by
 *     grid-wide barriers, each workgroup prefetching its next product's
 *     first weights into registers before the barrier (UNSUPPORTED if the
 *     largest activation exceeds 64 KB of LDS);
 *   2 one streaming persistent kernel per token: one workgroup per CU whose
 *     producer waves copy the weights of every product, in order, from HBM
 *     into an LDS ring while its consumer waves compute, so the weight
 *     stream runs through the grid barriers (UNSUPPORTED unless every K is a
 *     multiple of 64 and the activation plus the ring fit in LDS);
 *   3 the same producer/consumer workgroups as mode 2, one launch per
 *     product (four per layer, no grid barriers; same limits as mode 2).
 * Each output is the same dot product within the same bound; the summation
 * order, and so the low bits, differ between implementations.  INVALID_ARG
 * for another mode, STATE without resident layers, UNSUPPORTED for modes
 * 1-3 on a decoder with a KV cache. */
q4_status q4_decoder_set_persistent(void *dec, int32_t mode);
/* After the stream has completed a persistent step (mode 1 or 2): Q4_OK, or
 * Q4_ERR_HIP if a bounded wait (grid barrier, ring slot, ring space) gave up
 * (the step's results are then invalid; the flag is cleared).  Synchronous. */
q4_status q4_decoder_check(void *dec);
/* Runs all layers for one token.  ctx_len picks the context bucket: the
 * smallest of 512, 1024, 2048, 4096 that is >= ctx_len; the first call for a
 * bucket captures the layer loop into a HIP graph on `stream` (which must
 * not be the NULL stream), later calls replay it.  ctx_len <= 0 is
 * INVALID_ARG, ctx_len > 4096 is UNSUPPORTED.  Graphs bake in every pointer
 * of the description: those buffers must outlive the decoder.  With a KV
 * cache, ctx_len above max_ctx is INVALID_ARG; the call first enqueues the
 * write of the position word (ctx_len - 1), outside the graph, and the
 * graph's attention covers min(bucket, max_ctx) positions, of which those
 * past the position contribute nothing. */
q4_status decode_step_graph(void *dec, int32_t ctx_len, hipStream_t stream);
/* Same layer loop, enqueued eagerly without a graph (for checking); with a
 * KV cache at the context length of the last q4_decoder_set_context
 * (or decode_step_graph) call, 1 before any. */
q4_status q4_decode_step_eager(void *dec, hipStream_t stream);
/* Layer-wise profiling (PipeLLM, "Layer 2: Asynchronous Weight
 * Prefetching" lists per-layer analysis and event-based timing among its
 * tools): the eager step with a timing event recorded on `stream` after
 * every kernel.  Writes each kernel's duration in milliseconds to the host
 * array ms_out in launch order -- per layer: QKV (with the first norm), O,
 * gate+up (with the second norm and the SiLU gate), down: 4 per layer --
 * and their count to *n_out.  With a KV cache the attention kernels get a
 * mark of their own after QKV: 5 per layer.  capacity must be at least that
 * count times n_layers.
 * Synchronises `stream` before returning. */
q4_status q4_decode_step_profiled(void *dec, hipStream_t stream, float *ms_out,
                                  int32_t capacity, int32_t *n_out);
/* One layer, eagerly, with the weights given (e.g. a streamed slot).  With a
 * KV cache, layers driven one at a time must come in order 0..n_layers-1
 * per token (the cache slice follows that order); q4_decoder_set_context
 * or a completed token restarts it at layer 0. */
q4_status q4_decode_layer(void *dec, const q4_layer *layer, hipStream_t stream);
/* Decoders with a KV cache: sets the context length (1..max_ctx) of the
 * next eager step or layer-by-layer token and enqueues, on `stream`, the
 * write of the position word the attention kernels read.  decode_step_graph
 * does this itself.  Without a cache: STATE. */
q4_status q4_decoder_set_context(void *dec, int32_t ctx_len, hipStream_t stream);
/* One product of a layer, eagerly: which = 0 QKV (RMSNorm of h, V gather
 * into the attention output), 1 O (h += ...), 2 gate+up (RMSNorm of h, its
 * binary16 result kept in the workspace, SiLU gate into the MLP activation),
 * 3 down (h += ...).  With a KV cache, 0 is followed by attention over the
 * cache slice of the current layer (which advances after 3).  Calling 0..3
 * in order equals q4_decode_layer; single
 * products let a caller inspect every intermediate (the workspace sections
 * listed above).  INVALID_ARG for another index or bad shapes. */
q4_status q4_decode_layer_part(void *dec, const q4_layer *layer, int32_t which,
                               hipStream_t stream);
/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: one
 * decoder layer on the fp32 residual h (device f32[d_model], 16-byte
 * aligned, in/out) exactly as q4_decode_layer computes it on a decoder
 * without a KV cache (the same kernels, so the same bits), without a
 * decoder object or a workspace.  The four intermediates (normed
 * activation, QKV output, attention output, gated MLP activation) live in
 * a library-owned static device array of Q4_NOALLOC_SCRATCH_BYTES per GPU,
 * held until the process ends; the call allocates nothing, host or device.
 * Dimensions as in q4_model_desc; the layer's matrices must have the
 * decoder's shapes.  INVALID_ARG for bad dimensions, shapes or pointers;
 * UNSUPPORTED when the intermediates,
 *   align256(2 max(d_model, d_ff)) + align256(4 (n_heads + 2 n_kv_heads)
 *   head_dim) + align256(2 n_heads head_dim) + align256(2 d_ff) bytes,
 * exceed Q4_NOALLOC_SCRATCH_BYTES (the 70B shapes need 172,032).  Every
 * call on one GPU uses that GPU's single array: calls whose work overlaps
 * in time on one GPU (streams not ordered with each other) race.  Nothing
 * in the array needs to start at zero: each call writes every intermediate
 * before reading it, and the array keeps the last call's values. */
#define Q4_NOALLOC_SCRATCH_BYTES (256 * 1024)
q4_status q4_decode_layer_noalloc(const q4_layer *layer, int32_t d_model, int32_t n_heads,
                                  int32_t n_kv_heads, int32_t head_dim, int32_t d_ff,
                                  float eps, float *h, hipStream_t stream);
/* Verify step: the first B columns of h_batch (1 <= B <= max_batch), each
 * the residual of one token, go through all resident layers together: per
 * layer, per column RMSNorm to binary16, the QKV, O, gate+up and down
 * products as small-batch INT4 products of B columns (q4_gemm_smallbatch's
 * kernels; O and down add into h_batch), and the one-token glue between
 * them per column.  Column b ends exactly as if its token were decoded
 * alone, within the product bound (B = 1 runs the single-token kernels and
 * equals q4_decode_step_eager bitwise; two or three columns of a model
 * whose products all fit the vector-ALU batch kernel, with the RMSNorm in
 * the QKV and gate+up products' prologue, equal it bitwise as well).  With a KV cache the columns are draft
 * tokens at consecutive positions: column b at position ctx - 1 + b, ctx
 * the context length of the last q4_decoder_set_context; per layer all B
 * key/value rows are stored first, then every column attends causally over
 * rows 0..ctx - 1 + b (the earlier columns included).  Eager enqueue on
 * `stream`.  STATE without resident layers or without max_batch;
 * INVALID_ARG for B outside 1..max_batch or ctx + B - 1 above max_ctx;
 * UNSUPPORTED for ctx + B - 1 above 4096. */
q4_status q4_decode_verify_eager(void *dec, int32_t B, hipStream_t stream);
/* The same, captured once per B (and, with a KV cache, per context bucket
 * of ctx + B - 1) as a HIP graph on `stream` (not NULL) and replayed; the
 * position word is not part of the graph (q4_decoder_set_context writes
 * it). */
q4_status q4_decode_verify_graph(void *dec, int32_t B, hipStream_t stream);
/* Frees graphs and host state.  Call after the last step has completed. */
q4_status q4_decoder_destroy(void *dec);

/* ------------------------------------------------------------------ */
/* Layer weight streaming (PipeLLM, "Layer 2: Asynchronous Weight        */
/* Prefetching"; PIPO, "Method", "Pipeline design", "Data transfer suite") */
/* ------------------------------------------------------------------ */

/* One layer's four matrices merged into one blob (one copy per layer):
 * sections, in order, qkv.packed, qkv.scales, o.packed, o.scales,
 * gate_up.packed, gate_up.scales, down.packed, down.scales, each starting
 * at a 256-byte aligned offset.  shapes: host; only N and K are read.
 * offsets: host size_t[8]; bytes: host, total blob size. */
q4_status q4_layer_blob_layout(const q4_layer *shapes, size_t offsets[8],
                               size_t *bytes);
/* q4_layer whose pointers point into a blob at `base` (device). */
q4_status q4_layer_from_blob(const q4_layer *shapes, const void *base,
                             q4_layer *out);

typedef struct {
    int32_t n_layers;
    const void *const *host_blobs; /* host array [n_layers] of pinned host
                                      pointers (hipHostMalloc / pinned torch);
                                      may be NULL for resident layers */
    const size_t *blob_bytes;      /* host array [n_layers], every layer */
    void *slot[2];                 /* two device buffers of slot_bytes */
    size_t slot_bytes;             /* >= every blob_bytes[l] */
    hipStream_t copy;              /* copy stream, not NULL */
    /* Chunked transfer over two copy streams (PIPO, "Method", "Data
     * transfer suite": blockwise transfer, several transfer threads).
     * copy2: a second copy stream, or NULL for one.  chunk_bytes: a layer's
     * copy is split into pieces of this many bytes (multiple of 256),
     * alternating between the copy streams; 0 = one piece per layer. */
    hipStream_t copy2;
    size_t chunk_bytes;
    /* Partial residency (PIPO, "Method", "Automatic configuration" and the
     * performance / memory-efficient pipeline modes): host array
     * [n_layers] of device pointers, 256-byte aligned, each a blob of
     * layer l in q4_layer_blob_layout already in HBM; NULL entries (or a
     * NULL array) are streamed.  Resident layers are never copied; the
     * two slots serve only the streamed layers. */
    void *const *resident;
} q4_wstream_desc;

/* Copies the description and creates events; retains every pointer.
 * INVALID_ARG for a chunk size not a multiple of 256 or a misaligned
 * resident blob. */
q4_status q4_wstream_create(const q4_wstream_desc *d, void **ws);
/* Placement rule for partial residency (PIPO, "Method", "Automatic
 * configuration": its Eq. 1 is missing from the page; reading: keep
 * everything resident when it fits, else keep as many layers as the budget
 * holds after the two streaming slots, spread evenly over the depth).
 *   all n_layers * layer_bytes <= budget_bytes: every layer resident;
 *   else k = min(n_layers - 1, (budget_bytes - 2 * layer_bytes) /
 *   layer_bytes) layers resident, layer floor((2i + 1) * n_layers / (2k))
 *   for i < k; UNSUPPORTED if the budget holds less than the two slots.
 * resident: host int32[n_layers] out (1 resident, 0 streamed);
 * *n_resident: host out, their count.  Host-only, no GPU work. */
q4_status q4_offload_plan(int32_t n_layers, size_t layer_bytes, size_t budget_bytes,
                          int32_t *resident, int32_t *n_resident);
/* Starts the host->device copy of `layer` into the next slot (slots
 * alternate by call count); STATE for a resident layer.  If that slot was handed out by an earlier
 * weight_stream_wait, all work enqueued on that call's compute stream
 * before THIS call is treated as its last use: the copy waits for it.
 * STATE if the next slot holds a layer that was begun but not yet waited. */
q4_status weight_stream_begin(void *ws, int32_t layer);
/* Makes `compute` wait until `layer`'s copy has landed and returns its slot
 * (device pointer to the blob) in *slot_ptr.  Layers must be waited in the
 * order they were begun; STATE otherwise. */
q4_status weight_stream_wait(void *ws, int32_t layer, hipStream_t compute,
                             void **slot_ptr);
/* Destroys events.  Call after all enqueued work has completed. */
q4_status q4_wstream_destroy(void *ws);

/* One token of the decoder with its layers streamed through `ws`: the
 * first streamed layer is begun (unless already begun by the previous
 * token), then for each layer l in order: a resident layer is computed
 * from its blob; a streamed layer has the copy of the next streamed layer
 * (wrapping to the next token's first) begun before l is waited and
 * computed on `compute`.  The blob layout must be q4_layer_blob_layout of
 * the decoder's shapes.  With a KV cache layer l attends over cache slice
 * l at the context length set by q4_decoder_set_context.  Returns once the
 * previous call's work on `compute` has completed, so the host stays at
 * most one token ahead of the device (deeper queues of copies and
 * cross-stream waits made the copies slower). */
q4_status q4_decode_token_streamed(void *dec, void *ws, hipStream_t compute);

#ifdef __cplusplus
}
#endif

#endif /* Q4_H */
