// Per-token decode loop, its HIP-graph cache keyed by context bucket, and
// double-buffered layer streaming from pinned host memory.
//
// Graph capture: PipeLLM: Faster Local LLM Inference Than llama.cpp via
// System-Level Optimizations, "Layer 1: CUDA Graph Compilation" -- the
// decoding loop is captured once as a static graph, with context-length
// buckets 512/1024/2048/4096 and the graph chosen by sequence length (we take
// the smallest bucket that holds ctx_len).
//
// Streaming: same page, "Layer 2: Asynchronous Weight Prefetching" (separate
// compute and copy streams, pinned host buffers, double-buffered staging),
// and PIPO: Pipelined Offloading for Efficient Inference on Consumer
// Devices, "Method": "Pipeline design" (load the next layer, wait for the
// current layer's load, compute), "Two pipeline modes" (the performance mode
// keeps two layers on the GPU) and "Data transfer suite" (a layer's tensors
// merged into one transfer).  PIPO's three transfer threads become one copy
// stream plus events: a pinned host->device copy needs no host thread.
#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include "q4_internal.h"
#include "q4_persistent.h"
#include "q4_attention.h"
#include "q4_verify.h"

namespace q4 {
namespace {

constexpr int kBuckets[4] = {512, 1024, 2048, 4096};
constexpr int kKernelsPerLayer = 4;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Dims {
    int64_t d, H, Hkv, hd, dff, nqkv;
};

struct Decoder {
    q4_model_desc desc;
    std::vector<q4_layer> layers;
    Dims dims;
    uint16_t *a16 = nullptr; // f16[max(d, dff)] normed activation
    float *qkv = nullptr;    // f32[nqkv]
    uint16_t *oin = nullptr; // f16[H*hd]
    uint16_t *mlp = nullptr; // f16[dff]
    uint32_t *bar = nullptr; // grid-barrier words of the persistent kernel
    DevLayer *dev_layers = nullptr; // device copy of the layer table
    int32_t mode = 0; // 0 four kernels per layer, 1 persistent, 2 streaming persistent,
                      // 3 streaming workgroups, one launch per product
    hipGraphExec_t exec[4] = {nullptr, nullptr, nullptr, nullptr};
    // attention over the KV cache (kv == nullptr: one-token stand-in)
    uint16_t *kv = nullptr;
    int32_t *pos_dev = nullptr;  // position word the attention kernels read
    float *att_part = nullptr;   // per-chunk partials
    float *qrot = nullptr;       // rotated queries, f32 [max(1, max_batch)][H * hd]
    void *rope = nullptr;        // rotation table
    int32_t ctx = 1;             // context length of eager / layer-by-layer steps
    int32_t att_chunks = 1;      // chunks the attention kernels cover
    int32_t cursor = 0;          // next layer of a layer-by-layer token
    // batched verify step (max_batch columns)
    float *hb = nullptr;         // caller's f32[max_batch][d]
    uint16_t *xb = nullptr;      // f16[max_batch][d]
    float *qkvb = nullptr;       // f32[max_batch][nqkv]
    uint16_t *oinb = nullptr;    // f16[max_batch][H*hd]
    uint16_t *mlpb = nullptr;    // f16[max_batch][dff]
    hipGraphExec_t vexec[4][Q4_MAX_BATCH + 1] = {}; // [context bucket][B]
};

q4_status dims_of(const q4_model_desc *m, Dims *out) {
    if (!m)
        return fail(Q4_ERR_INVALID_ARG, "decoder: null description");
    if (m->n_layers < 1 || m->d_model < 32 || m->n_heads < 1 || m->n_kv_heads < 1 ||
        m->head_dim < 1 || m->d_ff < 32)
        return fail(Q4_ERR_INVALID_ARG, "decoder: non-positive or too small dimension");
    if (m->n_heads % m->n_kv_heads != 0)
        return fail(Q4_ERR_INVALID_ARG, "decoder: n_heads %% n_kv_heads != 0");
    if (!(m->eps >= 0.0f))
        return fail(Q4_ERR_INVALID_ARG, "decoder: eps must be >= 0");
    Dims d;
    d.d = m->d_model;
    d.H = m->n_heads;
    d.Hkv = m->n_kv_heads;
    d.hd = m->head_dim;
    d.dff = m->d_ff;
    d.nqkv = (d.H + 2 * d.Hkv) * d.hd;
    if (d.d % 32 || (d.H * d.hd) % 32 || d.dff % 32)
        return fail(Q4_ERR_INVALID_ARG,
                    "decoder: d_model, n_heads*head_dim and d_ff must be multiples of 32");
    if (m->kv_cache) {
        if (!aligned(m->kv_cache, 16))
            return fail(Q4_ERR_INVALID_ARG, "decoder: kv_cache not 16-byte aligned");
        if (m->max_ctx < 1 || m->max_ctx > (1 << 20))
            return fail(Q4_ERR_INVALID_ARG, "decoder: max_ctx %d outside 1..%d", m->max_ctx,
                        1 << 20);
        if (!(m->rope_base > 0.0f))
            return fail(Q4_ERR_INVALID_ARG, "decoder: rope_base must be > 0");
        if (!attention_supported(m->n_heads, m->n_kv_heads, m->head_dim))
            return fail(Q4_ERR_UNSUPPORTED,
                        "decoder: attention needs n_heads/n_kv_heads in {1,2,4,8} and head_dim "
                        "64 or 128");
    }
    if (m->max_batch < 0 || m->max_batch > Q4_MAX_BATCH)
        return fail(Q4_ERR_INVALID_ARG, "decoder: max_batch %d outside 0..%d", m->max_batch,
                    Q4_MAX_BATCH);
    *out = d;
    return Q4_OK;
}

// Bytes of the verify-step sections for `mb` columns.
size_t verify_bytes(const Dims &d, int32_t mb) {
    if (mb <= 0)
        return 0;
    return align256((size_t)mb * d.d * 2) + align256((size_t)mb * d.nqkv * 4) +
           align256((size_t)mb * d.H * d.hd * 2) + align256((size_t)mb * d.dff * 2);
}

size_t workspace_bytes(const Dims &d, int64_t n_layers, const q4_model_desc *m) {
    size_t b = align256(std::max(d.d, d.dff) * 2) + align256(d.nqkv * 4) +
               align256(d.H * d.hd * 2) + align256(d.dff * 2) + kBarBytes +
               align256((size_t)n_layers * sizeof(DevLayer));
    if (m && m->kv_cache)
        b += 256 +
             align256(attention_partial_bytes((int32_t)d.H, (int32_t)d.Hkv, (int32_t)d.hd,
                                              m->max_ctx) *
                      (size_t)std::max(1, m->max_batch)) +
             align256((size_t)d.H * d.hd * 4 * (size_t)std::max(1, m->max_batch)) +
             align256(rope_table_bytes(m->max_ctx, (int32_t)d.hd));
    if (m)
        b += verify_bytes(d, m->max_batch);
    return b;
}

void layer_shapes(const Dims &d, q4_layer *s) {
    *s = q4_layer{};
    s->qkv.N = d.nqkv;
    s->qkv.K = d.d;
    s->o.N = d.d;
    s->o.K = d.H * d.hd;
    s->gate_up.N = 2 * d.dff;
    s->gate_up.K = d.d;
    s->down.N = d.d;
    s->down.K = d.dff;
}

q4_status check_layer(const Dims &d, const q4_layer &L, int idx) {
    q4_layer want;
    layer_shapes(d, &want);
    const q4_matrix *got[4] = {&L.qkv, &L.o, &L.gate_up, &L.down};
    const q4_matrix *exp[4] = {&want.qkv, &want.o, &want.gate_up, &want.down};
    const char *names[4] = {"qkv", "o", "gate_up", "down"};
    for (int i = 0; i < 4; ++i) {
        if (got[i]->N != exp[i]->N || got[i]->K != exp[i]->K)
            return fail(Q4_ERR_INVALID_ARG, "decoder: layer %d %s is %lldx%lld, expected %lldx%lld",
                        idx, names[i], (long long)got[i]->N, (long long)got[i]->K,
                        (long long)exp[i]->N, (long long)exp[i]->K);
        Q4_CHECK(check_matrix(got[i]->packed, got[i]->scales, got[i]->N, got[i]->K, names[i]));
    }
    return Q4_OK;
}

// Records a timing mark on `s` after each kernel when profiling.
struct Marks {
    std::vector<hipEvent_t> *ev = nullptr;
    q4_status mark(hipStream_t s) {
        if (!ev)
            return Q4_OK;
        hipEvent_t e = nullptr;
        Q4_HIP(hipEventCreate(&e));
        ev->push_back(e);
        Q4_HIP(hipEventRecord(e, s));
        return Q4_OK;
    }
};

// The four kernels of a layer, in order.
enum Kern { kQkv = 0, kO = 1, kGateUp = 2, kDown = 3 };

// Attention of layer `layer` over its cache slice, after the QKV product:
// `batch` token columns of qkv (default: the single-token buffers).
q4_status enqueue_attention(Decoder *dec, int32_t layer, hipStream_t s, int32_t batch = 1,
                            const float *qkv = nullptr, uint16_t *out = nullptr,
                            bool rows_stored = false) {
    const Dims &d = dec->dims;
    const size_t S = (size_t)d.Hkv * (size_t)dec->desc.max_ctx * (size_t)d.hd;
    AttnArgs a{};
    a.qkv = qkv ? qkv : dec->qkv;
    a.kc = dec->kv + 2 * (size_t)layer * S;
    a.vc = a.kc + S;
    a.pos_dev = dec->pos_dev;
    a.max_ctx = dec->desc.max_ctx;
    a.H = (int32_t)d.H;
    a.Hkv = (int32_t)d.Hkv;
    a.hd = (int32_t)d.hd;
    a.rope = dec->rope;
    a.qrot = dec->qrot;
    a.part = dec->att_part;
    a.nchunk = dec->att_chunks;
    a.out = out ? out : dec->oin;
    a.batch = batch;
    a.rows_stored = rows_stored;
    return launch_attention(a, s);
}

// The QKV product of one token column with the first RMSNorm in its
// prologue: x the fp32 residual, y the fp32 QKV rows.  When attention over
// the cache slice of `layer` follows (a KV cache and layer >= 0), the
// epilogue also rotates the query heads into dec->qrot and stores the
// token's rotated key and its value, in binary16, into cache row
// *pos_dev; otherwise the V rows land, as binary16, in `oin` for every
// query head of their group (the one-token output).
q4_status launch_qkv(Decoder *dec, const q4_layer &L, int32_t layer, const float *x, float *y,
                     uint16_t *oin, hipStream_t s) {
    const Dims &d = dec->dims;
    EpiArgs ea{};
    ea.y = y;
    ea.hd = (int32_t)d.hd;
    ea.eps = dec->desc.eps;
    if (dec->kv && layer >= 0) {
        const size_t S = (size_t)d.Hkv * (size_t)dec->desc.max_ctx * (size_t)d.hd;
        ea.pos_dev = dec->pos_dev;
        ea.rope = static_cast<const float2 *>(dec->rope);
        ea.qrot = dec->qrot;
        ea.kc = dec->kv + 2 * (size_t)layer * S;
        ea.vc = ea.kc + S;
        ea.n_q_heads = (int32_t)d.H;
        ea.n_kv_heads = (int32_t)d.Hkv;
        ea.max_ctx = dec->desc.max_ctx;
        return launch_gemv(L.qkv.packed, L.qkv.scales, x, Pro::RmsNorm, L.qkv.N, L.qkv.K,
                           Epi::QkvRope, ea, s);
    }
    ea.out16 = oin;
    ea.v_off = (d.H + d.Hkv) * d.hd;
    ea.group = (int32_t)(d.H / d.Hkv);
    return launch_gemv(L.qkv.packed, L.qkv.scales, x, Pro::RmsNorm, L.qkv.N, L.qkv.K,
                       Epi::QkvGather, ea, s);
}

// One product of a layer; `layer` >= 0 names its cache slice: with a KV
// cache the QKV product prepares attention over that slice and, with
// `attention`, is followed by it (layer < 0: the product alone, for timing).
q4_status enqueue_kernel(Decoder *dec, const q4_layer &L, int32_t layer, int which,
                         hipStream_t s, bool attention = true) {
    const Dims &d = dec->dims;
    float *h = dec->desc.h;
    EpiArgs ea{};
    switch (which) {
    case kQkv:
        Q4_CHECK(launch_qkv(dec, L, layer, h, dec->qkv, dec->oin, s));
        if (dec->kv && layer >= 0 && attention)
            return enqueue_attention(dec, layer, s);
        return Q4_OK;
    case kO:
        ea.y = h;
        return launch_gemv(L.o.packed, L.o.scales, dec->oin, Pro::F16, L.o.N, L.o.K,
                           Epi::Residual, ea, s);
    case kGateUp:
        // gate+up with the second RMSNorm in its prologue and the SiLU gate
        // in its epilogue (rows j and dff + j meet in one 16-lane row).
        ea.out16 = dec->mlp;
        ea.pair_off = d.dff;
        ea.eps = dec->desc.eps;
        ea.norm_out = dec->a16;
        return launch_gemv(L.gate_up.packed, L.gate_up.scales, h, Pro::RmsNorm, L.gate_up.N,
                           L.gate_up.K, Epi::SiluPair, ea, s);
    case kDown:
        ea.y = h;
        return launch_gemv(L.down.packed, L.down.scales, dec->mlp, Pro::F16, L.down.N,
                           L.down.K, Epi::Residual, ea, s);
    }
    return fail(Q4_ERR_INVALID_ARG, "decoder: kernel index %d", which);
}

// Enqueue layer `layer` on `s`: four products (plus attention with a cache).
q4_status enqueue_layer(Decoder *dec, const q4_layer &L, int32_t layer, hipStream_t s,
                        Marks marks = {}) {
    for (int k = kQkv; k <= kDown; ++k) {
        Q4_CHECK(enqueue_kernel(dec, L, layer, k, s, false));
        Q4_CHECK(marks.mark(s));
        if (k == kQkv && dec->kv && layer >= 0) {
            Q4_CHECK(enqueue_attention(dec, layer, s));
            Q4_CHECK(marks.mark(s));
        }
    }
    return Q4_OK;
}

q4_status enqueue_all(Decoder *dec, hipStream_t s) {
    if (dec->mode != 0) {
        PersistArgs a{};
        a.layers = dec->dev_layers;
        a.n_layers = (int32_t)dec->layers.size();
        a.h = dec->desc.h;
        a.qkv = dec->qkv;
        a.oin = dec->oin;
        a.mlp = dec->mlp;
        a.norm_out = dec->a16;
        a.d = (int32_t)dec->dims.d;
        a.H = (int32_t)dec->dims.H;
        a.Hkv = (int32_t)dec->dims.Hkv;
        a.hd = (int32_t)dec->dims.hd;
        a.dff = (int32_t)dec->dims.dff;
        a.eps = dec->desc.eps;
        a.bar = dec->bar;
        if (dec->mode == 3) {
            for (int32_t l = 0; l < a.n_layers; ++l)
                for (int32_t k = 0; k < 4; ++k)
                    Q4_CHECK(launch_stream_product(a, l, k, s));
            return Q4_OK;
        }
        return dec->mode == 2 ? launch_stream(a, s) : launch_persistent(a, s);
    }
    for (size_t l = 0; l < dec->layers.size(); ++l)
        Q4_CHECK(enqueue_layer(dec, dec->layers[l], (int32_t)l, s));
    return Q4_OK;
}

// Verify step: B residual columns of dec->hb through every resident layer.
// B = 1 runs the single-token kernels on the batch buffers.
q4_status enqueue_verify(Decoder *dec, int32_t B, hipStream_t s) {
    const Dims &d = dec->dims;
    const float eps = dec->desc.eps;
    for (int32_t l = 0; l < (int32_t)dec->layers.size(); ++l) {
        const q4_layer &L = dec->layers[(size_t)l];
        if (B == 1) {
            Q4_CHECK(launch_qkv(dec, L, l, dec->hb, dec->qkvb, dec->oinb, s));
            if (dec->kv)
                Q4_CHECK(enqueue_attention(dec, l, s, 1, dec->qkvb, dec->oinb));
            EpiArgs ea{};
            ea.y = dec->hb;
            Q4_CHECK(launch_gemv(L.o.packed, L.o.scales, dec->oinb, Pro::F16, L.o.N, L.o.K,
                                 Epi::Residual, ea, s));
            ea = EpiArgs{};
            ea.out16 = dec->mlpb;
            ea.pair_off = d.dff;
            ea.eps = eps;
            ea.norm_out = dec->xb;
            Q4_CHECK(launch_gemv(L.gate_up.packed, L.gate_up.scales, dec->hb, Pro::RmsNorm,
                                 L.gate_up.N, L.gate_up.K, Epi::SiluPair, ea, s));
            ea = EpiArgs{};
            ea.y = dec->hb;
            Q4_CHECK(launch_gemv(L.down.packed, L.down.scales, dec->mlpb, Pro::F16, L.down.N,
                                 L.down.K, Epi::Residual, ea, s));
            continue;
        }
        // Two or three columns of K <= 4096: the QKV product normalises its
        // columns itself (one launch less), else a norm kernel first.
        const bool norm_qkv = batch_norm_fits(L.qkv.K, B);
        if (norm_qkv) {
            EpiArgs ea{};
            ea.y = dec->qkvb;
            ea.eps = eps;
            Q4_CHECK(launch_batch_norm_product(L.qkv.packed, L.qkv.scales, dec->hb, L.qkv.N,
                                               L.qkv.K, B, Epi::Store, ea, s));
        } else {
            Q4_CHECK(launch_rmsnorm_batch(dec->hb, dec->xb, B, (int32_t)d.d, eps, s));
        }
        if (dec->kv && norm_qkv) {
            Q4_CHECK(enqueue_attention(dec, l, s, B, dec->qkvb, dec->oinb, false));
        } else if (dec->kv) {
            // the QKV epilogue stores the columns' key and value rows and
            // rotated queries where the matrix-core row-tile launch runs
            const size_t S = (size_t)d.Hkv * (size_t)dec->desc.max_ctx * (size_t)d.hd;
            GRope rp;
            rp.pos_dev = dec->pos_dev;
            rp.rope = static_cast<const float2 *>(dec->rope);
            rp.qrot = dec->qrot;
            rp.kc = dec->kv + 2 * (size_t)l * S;
            rp.vc = rp.kc + S;
            rp.hd = (int32_t)d.hd;
            rp.nq = (int32_t)d.H;
            rp.nkv = (int32_t)d.Hkv;
            rp.max_ctx = dec->desc.max_ctx;
            bool stored = false;
            Q4_CHECK(launch_gemm_qkv_rope(L.qkv.packed, L.qkv.scales, dec->xb, dec->qkvb,
                                          L.qkv.N, L.qkv.K, B, rp, s, &stored));
            Q4_CHECK(enqueue_attention(dec, l, s, B, dec->qkvb, dec->oinb, stored));
        } else {
            if (!norm_qkv)
                Q4_CHECK(launch_gemm_mfma(L.qkv.packed, L.qkv.scales, dec->xb, dec->qkvb,
                                          L.qkv.N, L.qkv.K, B, s));
            Q4_CHECK(launch_gather_batch(dec->qkvb, dec->oinb, B, (int32_t)d.H, (int32_t)d.Hkv,
                                         (int32_t)d.hd, s));
        }
        Q4_CHECK(launch_gemm_mfma(L.o.packed, L.o.scales, dec->oinb, dec->hb, L.o.N, L.o.K, B, s,
                                  true));
        // gate+up likewise where its columns run on the vector ALU
        if (silu_pair_on_valu(d.dff, L.gate_up.K, B) && batch_norm_fits(L.gate_up.K, B)) {
            EpiArgs ea{};
            ea.out16 = dec->mlpb;
            ea.pair_off = d.dff;
            ea.eps = eps;
            Q4_CHECK(launch_batch_norm_product(L.gate_up.packed, L.gate_up.scales, dec->hb,
                                               L.gate_up.N, L.gate_up.K, B, Epi::SiluPair, ea,
                                               s));
        } else {
            Q4_CHECK(launch_rmsnorm_batch(dec->hb, dec->xb, B, (int32_t)d.d, eps, s));
            Q4_CHECK(launch_gemm_silu_pair(L.gate_up.packed, L.gate_up.scales, dec->xb,
                                           dec->mlpb, d.dff, L.gate_up.K, B, s));
        }
        Q4_CHECK(launch_gemm_mfma(L.down.packed, L.down.scales, dec->mlpb, dec->hb, L.down.N,
                                  L.down.K, B, s, true));
    }
    return Q4_OK;
}

q4_status check_verify(Decoder *dec, int32_t B, const char *what) {
    if (!dec)
        return fail(Q4_ERR_INVALID_ARG, "%s: null decoder", what);
    if (dec->layers.empty())
        return fail(Q4_ERR_STATE, "%s: decoder has no resident layers", what);
    if (dec->desc.max_batch < 1)
        return fail(Q4_ERR_STATE, "%s: decoder created without max_batch", what);
    if (B < 1 || B > dec->desc.max_batch)
        return fail(Q4_ERR_INVALID_ARG, "%s: B=%d outside 1..%d", what, B, dec->desc.max_batch);
    if (dec->kv && dec->ctx + B - 1 > dec->desc.max_ctx)
        return fail(Q4_ERR_INVALID_ARG, "%s: positions %d..%d beyond max_ctx %d", what,
                    dec->ctx - 1, dec->ctx + B - 2, dec->desc.max_ctx);
    if (dec->kv && dec->ctx + B - 1 > kBuckets[3])
        return fail(Q4_ERR_UNSUPPORTED, "%s: context %d above %d", what, dec->ctx + B - 1,
                    kBuckets[3]);
    return Q4_OK;
}

// ------------------------------------------------------------ streaming
enum SlotState { kEmpty = 0, kLoading = 1, kInUse = 2 };

struct WStream {
    int32_t n_layers = 0;
    std::vector<const void *> blobs;
    std::vector<size_t> bytes;
    void *slot[2] = {nullptr, nullptr};
    size_t slot_bytes = 0;
    hipStream_t copy = nullptr;
    hipStream_t copy2 = nullptr;       // second copy stream (chunked transfer), may be null
    size_t chunk = 0;                  // bytes per piece, 0 = whole blob
    std::vector<void *> resident;      // device blob per layer, null = streamed
    hipEvent_t loaded[2] = {nullptr, nullptr};
    hipEvent_t loaded2[2] = {nullptr, nullptr}; // on copy2
    hipEvent_t freed[2] = {nullptr, nullptr};
    int state[2] = {kEmpty, kEmpty};
    int32_t layer_in[2] = {-1, -1};
    hipStream_t consumer[2] = {nullptr, nullptr};
    int64_t n_begun = 0;
    int64_t n_waited = 0;
    // Copy timing (q4_wstream_set_timing): per timed begin, events where
    // the copy starts (after the wait for its slot) and ends, on each copy
    // stream (index 0: copy, 1: copy2).
    std::vector<hipEvent_t> t_start[2], t_end[2];
    int32_t n_timed = 0;
    // End of each q4_decode_token_streamed call on the compute stream: the
    // next call returns only after the previous token has completed.
    hipEvent_t tok_done[2] = {nullptr, nullptr};
    int64_t n_tokens = 0;
};

void free_timing(WStream *w) {
    for (int c = 0; c < 2; ++c) {
        for (hipEvent_t e : w->t_start[c])
            (void)hipEventDestroy(e);
        for (hipEvent_t e : w->t_end[c])
            (void)hipEventDestroy(e);
        w->t_start[c].clear();
        w->t_end[c].clear();
    }
    w->n_timed = 0;
}

void destroy_wstream(WStream *w) {
    for (int i = 0; i < 2; ++i) {
        if (w->loaded[i])
            (void)hipEventDestroy(w->loaded[i]);
        if (w->loaded2[i])
            (void)hipEventDestroy(w->loaded2[i]);
        if (w->freed[i])
            (void)hipEventDestroy(w->freed[i]);
        if (w->tok_done[i])
            (void)hipEventDestroy(w->tok_done[i]);
    }
    free_timing(w);
    delete w;
}

} // namespace
} // namespace q4

using q4::Decoder;
using q4::WStream;

extern "C" q4_status q4_decoder_workspace_bytes(const q4_model_desc *m, size_t *out) {
    q4::Dims d;
    Q4_CHECK(q4::dims_of(m, &d));
    if (!out)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_decoder_workspace_bytes: null out");
    *out = q4::workspace_bytes(d, m->n_layers, m);
    return Q4_OK;
}

extern "C" q4_status q4_decoder_create(const q4_model_desc *m, void **dec_out) {
    if (!dec_out)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_decoder_create: null out pointer");
    *dec_out = nullptr;
    q4::Dims d;
    Q4_CHECK(q4::dims_of(m, &d));
    if (!m->h || !q4::aligned(m->h, 16))
        return q4::fail(Q4_ERR_INVALID_ARG,
                        "q4_decoder_create: h null or not 16-byte aligned");
    if (m->max_batch > 0 && (!m->h_batch || !q4::aligned(m->h_batch, 16)))
        return q4::fail(Q4_ERR_INVALID_ARG,
                        "q4_decoder_create: h_batch null or not 16-byte aligned");
    if (!m->workspace || !q4::aligned(m->workspace, 256))
        return q4::fail(Q4_ERR_INVALID_ARG,
                        "q4_decoder_create: workspace null or not 256-byte aligned");
    if (m->workspace_bytes < q4::workspace_bytes(d, m->n_layers, m))
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_decoder_create: workspace of %zu bytes < %zu",
                        m->workspace_bytes, q4::workspace_bytes(d, m->n_layers, m));
    if (m->layers) {
        for (int32_t l = 0; l < m->n_layers; ++l)
            Q4_CHECK(q4::check_layer(d, m->layers[l], l));
    }
    Decoder *dec = new (std::nothrow) Decoder();
    if (!dec)
        return q4::fail(Q4_ERR_OOM, "q4_decoder_create: out of host memory");
    dec->desc = *m;
    dec->dims = d;
    if (m->layers)
        dec->layers.assign(m->layers, m->layers + m->n_layers);
    dec->desc.layers = nullptr;
    char *ws = static_cast<char *>(m->workspace);
    dec->a16 = reinterpret_cast<uint16_t *>(ws);
    ws += q4::align256(std::max(d.d, d.dff) * 2);
    dec->qkv = reinterpret_cast<float *>(ws);
    ws += q4::align256(d.nqkv * 4);
    dec->oin = reinterpret_cast<uint16_t *>(ws);
    ws += q4::align256(d.H * d.hd * 2);
    dec->mlp = reinterpret_cast<uint16_t *>(ws);
    ws += q4::align256(d.dff * 2);
    dec->bar = reinterpret_cast<uint32_t *>(ws);
    ws += q4::kBarBytes;
    dec->dev_layers = reinterpret_cast<q4::DevLayer *>(ws);
    ws += q4::align256((size_t)m->n_layers * sizeof(q4::DevLayer));
    if (m->kv_cache) {
        dec->kv = static_cast<uint16_t *>(m->kv_cache);
        dec->pos_dev = reinterpret_cast<int32_t *>(ws);
        ws += 256;
        dec->att_part = reinterpret_cast<float *>(ws);
        ws += q4::align256(q4::attention_partial_bytes((int32_t)d.H, (int32_t)d.Hkv,
                                                       (int32_t)d.hd, m->max_ctx) *
                           (size_t)std::max(1, m->max_batch));
        dec->qrot = reinterpret_cast<float *>(ws);
        ws += q4::align256((size_t)d.H * d.hd * 4 * (size_t)std::max(1, m->max_batch));
        dec->rope = ws;
        // context length 1 until the caller sets another; the rotation table
        q4_status st = q4::launch_rope_table(dec->rope, m->max_ctx, (int32_t)d.hd,
                                             m->rope_base, nullptr);
        if (st != Q4_OK) {
            delete dec;
            return st;
        }
        ws += q4::align256(q4::rope_table_bytes(m->max_ctx, (int32_t)d.hd));
        hipError_t e = hipMemset(dec->pos_dev, 0, 256);
        if (e == hipSuccess)
            e = hipDeviceSynchronize();
        if (e != hipSuccess) {
            delete dec;
            return q4::fail(Q4_ERR_HIP, "q4_decoder_create: position word: %s",
                            hipGetErrorString(e));
        }
    }
    if (m->max_batch > 0) {
        const size_t mb = (size_t)m->max_batch;
        dec->hb = m->h_batch;
        dec->xb = reinterpret_cast<uint16_t *>(ws);
        ws += q4::align256(mb * d.d * 2);
        dec->qkvb = reinterpret_cast<float *>(ws);
        ws += q4::align256(mb * d.nqkv * 4);
        dec->oinb = reinterpret_cast<uint16_t *>(ws);
        ws += q4::align256(mb * d.H * d.hd * 2);
        dec->mlpb = reinterpret_cast<uint16_t *>(ws);
    }
    if (m->layers) {
        // Resident layers: the persistent kernel reads a device copy of the
        // layer table and keeps its barrier words next to it.
        std::vector<q4::DevLayer> table(m->n_layers);
        for (int32_t l = 0; l < m->n_layers; ++l) {
            const q4_matrix *mm[4] = {&m->layers[l].qkv, &m->layers[l].o, &m->layers[l].gate_up,
                                      &m->layers[l].down};
            for (int i = 0; i < 4; ++i) {
                table[l].packed[i] = mm[i]->packed;
                table[l].scales[i] = mm[i]->scales;
            }
        }
        hipError_t e = hipMemset(dec->bar, 0, q4::kBarBytes);
        if (e == hipSuccess)
            e = hipMemcpy(dec->dev_layers, table.data(), table.size() * sizeof(q4::DevLayer),
                          hipMemcpyHostToDevice);
        if (e != hipSuccess) {
            delete dec;
            return q4::fail(Q4_ERR_HIP, "q4_decoder_create: workspace setup: %s",
                            hipGetErrorString(e));
        }
        // Four kernels per layer by default: on MI355X they stream the
        // weights faster than the persistent kernel's barrier-separated
        // phases; the persistent step is opt-in.
        dec->mode = 0;
    }
    *dec_out = dec;
    return Q4_OK;
}

extern "C" q4_status q4_decode_step_eager(void *decp, hipStream_t stream) {
    Decoder *dec = static_cast<Decoder *>(decp);
    if (!dec)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_decode_step_eager: null decoder");
    if (dec->layers.empty())
        return q4::fail(Q4_ERR_STATE, "q4_decode_step_eager: decoder has no resident layers");
    dec->att_chunks = q4::attention_chunks(dec->ctx);
    return q4::enqueue_all(dec, stream);
}

extern "C" q4_status decode_step_graph(void *decp, int32_t ctx_len, hipStream_t stream) {
    Decoder *dec = static_cast<Decoder *>(decp);
    if (!dec)
        return q4::fail(Q4_ERR_INVALID_ARG, "decode_step_graph: null decoder");
    if (ctx_len <= 0)
        return q4::fail(Q4_ERR_INVALID_ARG, "decode_step_graph: ctx_len=%d <= 0", ctx_len);
    if (ctx_len > q4::kBuckets[3])
        return q4::fail(Q4_ERR_UNSUPPORTED, "decode_step_graph: ctx_len=%d above %d", ctx_len,
                        q4::kBuckets[3]);
    if (!stream)
        return q4::fail(Q4_ERR_INVALID_ARG, "decode_step_graph: capture needs a non-NULL stream");
    if (dec->layers.empty())
        return q4::fail(Q4_ERR_STATE, "decode_step_graph: decoder has no resident layers");
    if (dec->kv && ctx_len > dec->desc.max_ctx)
        return q4::fail(Q4_ERR_INVALID_ARG, "decode_step_graph: ctx_len=%d above max_ctx %d",
                        ctx_len, dec->desc.max_ctx);
    int b = 0;
    while (q4::kBuckets[b] < ctx_len)
        ++b;
    if (dec->kv) {
        // The position word sits outside the graph: one graph per bucket
        // serves every context length in it.
        Q4_CHECK(q4::launch_set_pos(dec->pos_dev, ctx_len - 1, stream));
        dec->ctx = ctx_len;
        dec->cursor = 0;
    }
    if (!dec->exec[b]) {
        dec->att_chunks = q4::attention_chunks(std::min(q4::kBuckets[b], dec->desc.max_ctx));
        Q4_HIP(hipStreamBeginCapture(stream, hipStreamCaptureModeThreadLocal));
        q4_status st = q4::enqueue_all(dec, stream);
        hipGraph_t graph = nullptr;
        hipError_t e = hipStreamEndCapture(stream, &graph);
        if (st != Q4_OK) {
            if (graph)
                (void)hipGraphDestroy(graph);
            return st;
        }
        if (e != hipSuccess)
            return q4::fail(Q4_ERR_HIP, "decode_step_graph: end capture: %s",
                            hipGetErrorString(e));
        hipGraphExec_t exec = nullptr;
        e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
        (void)hipGraphDestroy(graph);
        if (e != hipSuccess)
            return q4::fail(Q4_ERR_HIP, "decode_step_graph: instantiate: %s",
                            hipGetErrorString(e));
        dec->exec[b] = exec;
    }
    Q4_HIP(hipGraphLaunch(dec->exec[b], stream));
    return Q4_OK;
}

extern "C" q4_status q4_decode_layer(void *decp, const q4_layer *layer, hipStream_t stream) {
    Decoder *dec = static_cast<Decoder *>(decp);
    if (!dec || !layer)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_decode_layer: null decoder or layer");
    Q4_CHECK(q4::check_layer(dec->dims, *layer, -1));
    dec->att_chunks = q4::attention_chunks(dec->ctx);
    Q4_CHECK(q4::enqueue_layer(dec, *layer, dec->cursor, stream));
    dec->cursor = (dec->cursor + 1) % dec->desc.n_layers;
    return Q4_OK;
}

extern "C" q4_status q4_decode_layer_part(void *decp, const q4_layer *layer, int32_t which,
                                          hipStream_t stream) {
    Decoder *dec = static_cast<Decoder *>(decp);
    if (!dec || !layer)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_decode_layer_part: null decoder or layer");
    if (which < q4::kQkv || which > q4::kDown)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_decode_layer_part: product index %d", which);
    Q4_CHECK(q4::check_layer(dec->dims, *layer, -1));
    dec->att_chunks = q4::attention_chunks(dec->ctx);
    Q4_CHECK(q4::enqueue_kernel(dec, *layer, dec->cursor, which, stream));
    if (which == q4::kDown)
        dec->cursor = (dec->cursor + 1) % dec->desc.n_layers;
    return Q4_OK;
}

extern "C" q4_status q4_decoder_set_context(void *decp, int32_t ctx_len, hipStream_t stream) {
    Decoder *dec = static_cast<Decoder *>(decp);
    if (!dec)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_decoder_set_context: null decoder");
    if (!dec->kv)
        return q4::fail(Q4_ERR_STATE, "q4_decoder_set_context: decoder has no KV cache");
    if (ctx_len < 1 || ctx_len > dec->desc.max_ctx)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_decoder_set_context: ctx_len=%d outside 1..%d",
                        ctx_len, dec->desc.max_ctx);
    Q4_CHECK(q4::launch_set_pos(dec->pos_dev, ctx_len - 1, stream));
    dec->ctx = ctx_len;
    dec->cursor = 0;
    return Q4_OK;
}

extern "C" q4_status q4_decode_verify_eager(void *decp, int32_t B, hipStream_t stream) {
    Decoder *dec = static_cast<Decoder *>(decp);
    Q4_CHECK(q4::check_verify(dec, B, "q4_decode_verify_eager"));
    dec->att_chunks = q4::attention_chunks(dec->ctx + B - 1);
    return q4::enqueue_verify(dec, B, stream);
}

extern "C" q4_status q4_decode_verify_graph(void *decp, int32_t B, hipStream_t stream) {
    Decoder *dec = static_cast<Decoder *>(decp);
    Q4_CHECK(q4::check_verify(dec, B, "q4_decode_verify_graph"));
    if (!stream)
        return q4::fail(Q4_ERR_INVALID_ARG,
                        "q4_decode_verify_graph: capture needs a non-NULL stream");
    int bk = 0;
    if (dec->kv)
        while (q4::kBuckets[bk] < dec->ctx + B - 1)
            ++bk;
    if (!dec->vexec[bk][B]) {
        if (dec->kv)
            dec->att_chunks =
                q4::attention_chunks(std::min(q4::kBuckets[bk], dec->desc.max_ctx));
        Q4_HIP(hipStreamBeginCapture(stream, hipStreamCaptureModeThreadLocal));
        q4_status st = q4::enqueue_verify(dec, B, stream);
        hipGraph_t graph = nullptr;
        hipError_t e = hipStreamEndCapture(stream, &graph);
        if (st != Q4_OK) {
            if (graph)
                (void)hipGraphDestroy(graph);
            return st;
        }
        if (e != hipSuccess)
            return q4::fail(Q4_ERR_HIP, "q4_decode_verify_graph: end capture: %s",
                            hipGetErrorString(e));
        hipGraphExec_t exec = nullptr;
        e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
        (void)hipGraphDestroy(graph);
        if (e != hipSuccess)
            return q4::fail(Q4_ERR_HIP, "q4_decode_verify_graph: instantiate: %s",
                            hipGetErrorString(e));
        dec->vexec[bk][B] = exec;
    }
    Q4_HIP(hipGraphLaunch(dec->vexec[bk][B], stream));
    return Q4_OK;
}

extern "C" q4_status q4_decoder_destroy(void *decp) {
    Decoder *dec = static_cast<Decoder *>(decp);
    if (!dec)
        return Q4_OK;
    for (auto &e : dec->exec)
        if (e)
            (void)hipGraphExecDestroy(e);
    for (auto &row : dec->vexec)
        for (auto &e : row)
            if (e)
                (void)hipGraphExecDestroy(e);
    delete dec;
    return Q4_OK;
}

// ---------------------------------------------------------------- blobs
extern "C" q4_status q4_layer_blob_layout(const q4_layer *shapes, size_t offsets[8],
                                          size_t *bytes) {
    if (!shapes || !offsets || !bytes)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_layer_blob_layout: null argument");
    const q4_matrix *m[4] = {&shapes->qkv, &shapes->o, &shapes->gate_up, &shapes->down};
    size_t off = 0;
    for (int i = 0; i < 4; ++i) {
        if (m[i]->N < 1 || m[i]->K < 32 || m[i]->K % 32)
            return q4::fail(Q4_ERR_INVALID_ARG, "q4_layer_blob_layout: bad shape %d", i);
        offsets[2 * i] = off;
        off = q4::align256(off + (size_t)m[i]->N * (size_t)m[i]->K / 2);
        offsets[2 * i + 1] = off;
        off = q4::align256(off + (size_t)m[i]->N * (size_t)(m[i]->K / 32) * 2);
    }
    *bytes = off;
    return Q4_OK;
}

extern "C" q4_status q4_layer_from_blob(const q4_layer *shapes, const void *base,
                                        q4_layer *out) {
    if (!base || !out)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_layer_from_blob: null argument");
    size_t off[8], bytes;
    Q4_CHECK(q4_layer_blob_layout(shapes, off, &bytes));
    const char *b = static_cast<const char *>(base);
    q4_layer L = *shapes;
    q4_matrix *m[4] = {&L.qkv, &L.o, &L.gate_up, &L.down};
    for (int i = 0; i < 4; ++i) {
        m[i]->packed = reinterpret_cast<const uint8_t *>(b + off[2 * i]);
        m[i]->scales = reinterpret_cast<const uint16_t *>(b + off[2 * i + 1]);
    }
    *out = L;
    return Q4_OK;
}

// ------------------------------------------------------------- wstream
extern "C" q4_status q4_wstream_create(const q4_wstream_desc *d, void **ws_out) {
    if (!d || !ws_out)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_wstream_create: null argument");
    *ws_out = nullptr;
    if (d->n_layers < 1 || !d->host_blobs || !d->blob_bytes)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_wstream_create: need n_layers >= 1 and arrays");
    if (!d->slot[0] || !d->slot[1] || !d->copy)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_wstream_create: null slot or copy stream");
    if (!q4::aligned(d->slot[0], 256) || !q4::aligned(d->slot[1], 256))
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_wstream_create: slots must be 256-byte aligned");
    if (d->chunk_bytes % 256 != 0)
        return q4::fail(Q4_ERR_INVALID_ARG,
                        "q4_wstream_create: chunk_bytes %zu not a multiple of 256", d->chunk_bytes);
    for (int32_t l = 0; l < d->n_layers; ++l) {
        if (d->resident && d->resident[l]) {
            if (!q4::aligned(d->resident[l], 256))
                return q4::fail(Q4_ERR_INVALID_ARG,
                                "q4_wstream_create: resident blob %d not 256-byte aligned", l);
            continue;
        }
        if (!d->host_blobs[l])
            return q4::fail(Q4_ERR_INVALID_ARG, "q4_wstream_create: null blob %d", l);
        if (d->blob_bytes[l] > d->slot_bytes)
            return q4::fail(Q4_ERR_INVALID_ARG,
                            "q4_wstream_create: blob %d (%zu bytes) larger than a slot (%zu)", l,
                            d->blob_bytes[l], d->slot_bytes);
    }
    WStream *w = new (std::nothrow) WStream();
    if (!w)
        return q4::fail(Q4_ERR_OOM, "q4_wstream_create: out of host memory");
    w->n_layers = d->n_layers;
    w->blobs.assign(d->host_blobs, d->host_blobs + d->n_layers);
    w->bytes.assign(d->blob_bytes, d->blob_bytes + d->n_layers);
    w->slot[0] = d->slot[0];
    w->slot[1] = d->slot[1];
    w->slot_bytes = d->slot_bytes;
    w->copy = d->copy;
    w->copy2 = d->copy2;
    w->chunk = d->chunk_bytes;
    w->resident.assign((size_t)d->n_layers, nullptr);
    if (d->resident)
        for (int32_t l = 0; l < d->n_layers; ++l)
            w->resident[l] = d->resident[l];
    for (int i = 0; i < 2; ++i) {
        hipError_t e1 = hipEventCreateWithFlags(&w->loaded[i], hipEventDisableTiming);
        hipError_t e2 = hipEventCreateWithFlags(&w->freed[i], hipEventDisableTiming);
        hipError_t e3 = hipEventCreateWithFlags(&w->loaded2[i], hipEventDisableTiming);
        hipError_t e4 = hipEventCreateWithFlags(&w->tok_done[i], hipEventDisableTiming);
        if (e1 != hipSuccess || e2 != hipSuccess || e3 != hipSuccess || e4 != hipSuccess) {
            q4::destroy_wstream(w);
            return q4::fail(Q4_ERR_HIP, "q4_wstream_create: event creation failed");
        }
    }
    *ws_out = w;
    return Q4_OK;
}

extern "C" q4_status weight_stream_begin(void *wsp, int32_t layer) {
    WStream *w = static_cast<WStream *>(wsp);
    if (!w)
        return q4::fail(Q4_ERR_INVALID_ARG, "weight_stream_begin: null stream object");
    if (layer < 0 || layer >= w->n_layers)
        return q4::fail(Q4_ERR_INVALID_ARG, "weight_stream_begin: layer %d out of range", layer);
    if (w->resident[layer])
        return q4::fail(Q4_ERR_STATE, "weight_stream_begin: layer %d is resident", layer);
    const int s = (int)(w->n_begun & 1);
    if (w->state[s] == q4::kLoading)
        return q4::fail(Q4_ERR_STATE,
                        "weight_stream_begin: slot %d still holds layer %d, begun but not waited",
                        s, w->layer_in[s]);
    if (w->state[s] == q4::kInUse) {
        // Everything enqueued so far on the consumer stream is the last use
        // of this slot: the copy may overwrite it only after that work.
        Q4_HIP(hipEventRecord(w->freed[s], w->consumer[s]));
        Q4_HIP(hipStreamWaitEvent(w->copy, w->freed[s], 0));
        if (w->copy2)
            Q4_HIP(hipStreamWaitEvent(w->copy2, w->freed[s], 0));
    }
    const size_t total = w->bytes[layer];
    const size_t piece = w->chunk ? w->chunk : total;
    char *dst = static_cast<char *>(w->slot[s]);
    const char *src = static_cast<const char *>(w->blobs[layer]);
    const bool timed = w->n_timed < (int32_t)w->t_start[0].size();
    if (timed) {
        Q4_HIP(hipEventRecord(w->t_start[0][w->n_timed], w->copy));
        if (w->copy2)
            Q4_HIP(hipEventRecord(w->t_start[1][w->n_timed], w->copy2));
    }
    int k = 0;
    for (size_t off = 0; off < total; off += piece, ++k) {
        const size_t n = std::min(piece, total - off);
        hipStream_t cs = (w->copy2 && (k & 1)) ? w->copy2 : w->copy;
        Q4_HIP(hipMemcpyAsync(dst + off, src + off, n, hipMemcpyHostToDevice, cs));
    }
    Q4_HIP(hipEventRecord(w->loaded[s], w->copy));
    if (w->copy2)
        Q4_HIP(hipEventRecord(w->loaded2[s], w->copy2));
    if (timed) {
        Q4_HIP(hipEventRecord(w->t_end[0][w->n_timed], w->copy));
        if (w->copy2)
            Q4_HIP(hipEventRecord(w->t_end[1][w->n_timed], w->copy2));
        ++w->n_timed;
    }
    w->state[s] = q4::kLoading;
    w->layer_in[s] = layer;
    w->consumer[s] = nullptr;
    ++w->n_begun;
    return Q4_OK;
}

extern "C" q4_status weight_stream_wait(void *wsp, int32_t layer, hipStream_t compute,
                                        void **slot_ptr) {
    WStream *w = static_cast<WStream *>(wsp);
    if (!w || !slot_ptr)
        return q4::fail(Q4_ERR_INVALID_ARG, "weight_stream_wait: null argument");
    if (layer < 0 || layer >= w->n_layers)
        return q4::fail(Q4_ERR_INVALID_ARG, "weight_stream_wait: layer %d out of range", layer);
    const int s = (int)(w->n_waited & 1);
    if (w->state[s] != q4::kLoading || w->layer_in[s] != layer)
        return q4::fail(Q4_ERR_STATE, "weight_stream_wait: layer %d is not the next begun layer",
                        layer);
    Q4_HIP(hipStreamWaitEvent(compute, w->loaded[s], 0));
    if (w->copy2)
        Q4_HIP(hipStreamWaitEvent(compute, w->loaded2[s], 0));
    w->state[s] = q4::kInUse;
    w->consumer[s] = compute;
    ++w->n_waited;
    *slot_ptr = w->slot[s];
    return Q4_OK;
}

extern "C" q4_status q4_wstream_set_timing(void *wsp, int32_t capacity) {
    WStream *w = static_cast<WStream *>(wsp);
    if (!w || capacity < 0)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_wstream_set_timing: null stream or capacity < 0");
    q4::free_timing(w);
    const int nc = w->copy2 ? 2 : 1;
    for (int c = 0; c < nc; ++c) {
        w->t_start[c].assign((size_t)capacity, nullptr);
        w->t_end[c].assign((size_t)capacity, nullptr);
        for (int32_t i = 0; i < capacity; ++i) {
            if (hipEventCreate(&w->t_start[c][i]) != hipSuccess ||
                hipEventCreate(&w->t_end[c][i]) != hipSuccess) {
                q4::free_timing(w);
                return q4::fail(Q4_ERR_HIP, "q4_wstream_set_timing: event creation failed");
            }
        }
    }
    if (nc == 1) {
        w->t_start[1].clear();
        w->t_end[1].clear();
    }
    return Q4_OK;
}

extern "C" q4_status q4_wstream_copy_times(void *wsp, float *start_ms, float *end_ms,
                                           int32_t capacity, int32_t *n_out) {
    WStream *w = static_cast<WStream *>(wsp);
    if (!w || !start_ms || !end_ms || !n_out)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_wstream_copy_times: null argument");
    const int32_t n = std::min(capacity, w->n_timed);
    *n_out = 0;
    if (n <= 0)
        return Q4_OK;
    Q4_HIP(hipEventSynchronize(w->t_end[0][n - 1]));
    if (!w->t_end[1].empty())
        Q4_HIP(hipEventSynchronize(w->t_end[1][n - 1]));
    const hipEvent_t ref = w->t_start[0][0];
    for (int32_t i = 0; i < n; ++i) {
        float s = 0.0f, e = 0.0f;
        Q4_HIP(hipEventElapsedTime(&s, ref, w->t_start[0][i]));
        Q4_HIP(hipEventElapsedTime(&e, ref, w->t_end[0][i]));
        if (!w->t_start[1].empty()) {
            float s2 = 0.0f, e2 = 0.0f;
            Q4_HIP(hipEventElapsedTime(&s2, ref, w->t_start[1][i]));
            Q4_HIP(hipEventElapsedTime(&e2, ref, w->t_end[1][i]));
            s = std::min(s, s2);
            e = std::max(e, e2);
        }
        start_ms[i] = s;
        end_ms[i] = e;
    }
    *n_out = n;
    return Q4_OK;
}

extern "C" q4_status q4_offload_plan(int32_t n_layers, size_t layer_bytes, size_t budget_bytes,
                                     int32_t *resident, int32_t *n_resident) {
    if (n_layers < 1 || layer_bytes == 0 || !resident || !n_resident)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_offload_plan: need n_layers >= 1, layer_bytes > 0 "
                                            "and output arrays");
    for (int32_t l = 0; l < n_layers; ++l)
        resident[l] = 0;
    if (budget_bytes / layer_bytes >= (size_t)n_layers) {
        for (int32_t l = 0; l < n_layers; ++l)
            resident[l] = 1;
        *n_resident = n_layers;
        return Q4_OK;
    }
    if (budget_bytes / layer_bytes < 2)
        return q4::fail(Q4_ERR_UNSUPPORTED,
                        "q4_offload_plan: budget of %zu bytes holds fewer than the two slots",
                        budget_bytes);
    const int64_t k = std::min<int64_t>(n_layers - 1, (int64_t)(budget_bytes / layer_bytes) - 2);
    for (int64_t i = 0; i < k; ++i)
        resident[(2 * i + 1) * n_layers / (2 * k)] = 1;
    *n_resident = (int32_t)k;
    return Q4_OK;
}

extern "C" q4_status q4_wstream_destroy(void *wsp) {
    if (wsp)
        q4::destroy_wstream(static_cast<WStream *>(wsp));
    return Q4_OK;
}

extern "C" q4_status q4_decode_token_streamed(void *decp, void *wsp, hipStream_t compute) {
    Decoder *dec = static_cast<Decoder *>(decp);
    WStream *w = static_cast<WStream *>(wsp);
    if (!dec || !w)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_decode_token_streamed: null argument");
    if (w->n_layers != dec->desc.n_layers)
        return q4::fail(Q4_ERR_INVALID_ARG,
                        "q4_decode_token_streamed: stream has %d layers, decoder %d",
                        w->n_layers, dec->desc.n_layers);
    q4_layer shapes;
    q4::layer_shapes(dec->dims, &shapes);
    size_t off[8], bytes;
    Q4_CHECK(q4_layer_blob_layout(&shapes, off, &bytes));
    for (int32_t l = 0; l < w->n_layers; ++l)
        if (w->bytes[l] < bytes)
            return q4::fail(Q4_ERR_INVALID_ARG,
                            "q4_decode_token_streamed: blob %d has %zu bytes, layout needs %zu", l,
                            w->bytes[l], bytes);
    const int L = w->n_layers;
    dec->att_chunks = q4::attention_chunks(dec->ctx);
    std::vector<int32_t> streamed;
    for (int l = 0; l < L; ++l)
        if (!w->resident[l])
            streamed.push_back(l);
    const int S = (int)streamed.size();
    if (S > 0) {
        const int s0 = (int)(w->n_waited & 1);
        const bool prefetched =
            w->state[s0] == q4::kLoading && w->layer_in[s0] == streamed[0];
        if (!prefetched)
            Q4_CHECK(weight_stream_begin(w, streamed[0]));
    }
    int j = 0; // position of the next streamed layer
    for (int l = 0; l < L; ++l) {
        q4_layer layer;
        if (w->resident[l]) {
            Q4_CHECK(q4_layer_from_blob(&shapes, w->resident[l], &layer));
        } else {
            // The copy of the following streamed layer (after the last: the
            // next token's first) overlaps this layer's compute and that of
            // the resident layers in between.
            Q4_CHECK(weight_stream_begin(w, streamed[(j + 1) % S]));
            void *slot = nullptr;
            Q4_CHECK(weight_stream_wait(w, l, compute, &slot));
            Q4_CHECK(q4_layer_from_blob(&shapes, slot, &layer));
            ++j;
        }
        Q4_CHECK(q4::enqueue_layer(dec, layer, l, compute));
    }
    // Keep the host at most one token ahead of the device: wait for the
    // previous token's work before returning.  With several tokens of copies
    // and cross-stream waits queued the copies themselves ran slower
    // (70B shapes: 688-737 ms per token against 677 with this bound).
    Q4_HIP(hipEventRecord(w->tok_done[w->n_tokens & 1], compute));
    if (w->n_tokens > 0)
        Q4_HIP(hipEventSynchronize(w->tok_done[(w->n_tokens - 1) & 1]));
    ++w->n_tokens;
    return Q4_OK;
}

extern "C" q4_status q4_decode_step_profiled(void *decp, hipStream_t stream, float *ms_out,
                                             int32_t capacity, int32_t *n_out) {
    Decoder *dec = static_cast<Decoder *>(decp);
    if (!dec || !ms_out || !n_out)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_decode_step_profiled: null argument");
    if (dec->layers.empty())
        return q4::fail(Q4_ERR_STATE, "q4_decode_step_profiled: decoder has no resident layers");
    const int64_t need =
        (int64_t)dec->layers.size() * (q4::kKernelsPerLayer + (dec->kv ? 1 : 0));
    if (capacity < need)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_decode_step_profiled: capacity %d < %lld",
                        capacity, (long long)need);
    dec->att_chunks = q4::attention_chunks(dec->ctx);
    std::vector<hipEvent_t> ev;
    q4::Marks marks;
    marks.ev = &ev;
    q4_status st = marks.mark(stream);
    for (size_t l = 0; st == Q4_OK && l < dec->layers.size(); ++l)
        st = q4::enqueue_layer(dec, dec->layers[l], (int32_t)l, stream, marks);
    hipError_t e = hipStreamSynchronize(stream);
    if (st == Q4_OK && e != hipSuccess)
        st = q4::fail(Q4_ERR_HIP, "q4_decode_step_profiled: %s", hipGetErrorString(e));
    int32_t n = 0;
    for (size_t i = 1; st == Q4_OK && i < ev.size(); ++i) {
        float ms = 0.0f;
        e = hipEventElapsedTime(&ms, ev[i - 1], ev[i]);
        if (e != hipSuccess)
            st = q4::fail(Q4_ERR_HIP, "q4_decode_step_profiled: elapsed: %s",
                          hipGetErrorString(e));
        ms_out[n++] = ms;
    }
    for (hipEvent_t x : ev)
        (void)hipEventDestroy(x);
    *n_out = n;
    return st;
}

extern "C" q4_status q4_decode_kernel_time(void *decp, int32_t which, int32_t reps,
                                           hipStream_t stream, float *avg_us) {
    Decoder *dec = static_cast<Decoder *>(decp);
    if (!dec || !avg_us)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_decode_kernel_time: null argument");
    if (dec->layers.empty())
        return q4::fail(Q4_ERR_STATE, "q4_decode_kernel_time: decoder has no resident layers");
    if (which < 0 || which > 3 || reps < 1)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_decode_kernel_time: which=%d reps=%d", which,
                        reps);
    hipEvent_t e0 = nullptr, e1 = nullptr;
    Q4_HIP(hipEventCreate(&e0));
    hipError_t e = hipEventCreate(&e1);
    if (e != hipSuccess) {
        (void)hipEventDestroy(e0);
        return q4::fail(Q4_ERR_HIP, "q4_decode_kernel_time: %s", hipGetErrorString(e));
    }
    q4_status st = Q4_OK;
    const size_t L = dec->layers.size();
    if (hipEventRecord(e0, stream) != hipSuccess)
        st = q4::fail(Q4_ERR_HIP, "q4_decode_kernel_time: event record failed");
    for (int32_t i = 0; st == Q4_OK && i < reps; ++i)
        st = q4::enqueue_kernel(dec, dec->layers[(size_t)i % L], -1, which, stream);
    if (st == Q4_OK && hipEventRecord(e1, stream) != hipSuccess)
        st = q4::fail(Q4_ERR_HIP, "q4_decode_kernel_time: event record failed");
    if (st == Q4_OK && (e = hipEventSynchronize(e1)) != hipSuccess)
        st = q4::fail(Q4_ERR_HIP, "q4_decode_kernel_time: %s", hipGetErrorString(e));
    float ms = 0.0f;
    if (st == Q4_OK && (e = hipEventElapsedTime(&ms, e0, e1)) != hipSuccess)
        st = q4::fail(Q4_ERR_HIP, "q4_decode_kernel_time: %s", hipGetErrorString(e));
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (st == Q4_OK)
        *avg_us = ms * 1000.0f / (float)reps;
    return st;
}

extern "C" q4_status q4_decoder_set_persistent(void *decp, int32_t mode) {
    Decoder *dec = static_cast<Decoder *>(decp);
    if (!dec)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_decoder_set_persistent: null decoder");
    if (mode < 0 || mode > 3)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_decoder_set_persistent: mode %d", mode);
    if (mode != 0 && dec->layers.empty())
        return q4::fail(Q4_ERR_STATE, "q4_decoder_set_persistent: no resident layers");
    if (mode != 0 && dec->kv)
        return q4::fail(Q4_ERR_UNSUPPORTED,
                        "q4_decoder_set_persistent: persistent steps have no attention");
    const int32_t d = (int32_t)dec->dims.d, H = (int32_t)dec->dims.H,
                  hd = (int32_t)dec->dims.hd, dff = (int32_t)dec->dims.dff;
    if (mode == 1 && q4::persistent_lds_bytes(d, H, hd, dff) > 65536)
        return q4::fail(Q4_ERR_UNSUPPORTED, "q4_decoder_set_persistent: activations exceed LDS");
    if (mode == 2 || mode == 3)
        Q4_CHECK(q4::stream_supported(d, H, hd, dff, nullptr));
    if (mode != dec->mode) {
        for (auto &e : dec->exec)
            if (e) {
                (void)hipGraphExecDestroy(e);
                e = nullptr;
            }
        dec->mode = mode;
    }
    return Q4_OK;
}

extern "C" q4_status q4_decoder_check(void *decp) {
    Decoder *dec = static_cast<Decoder *>(decp);
    if (!dec)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_decoder_check: null decoder");
    if (dec->layers.empty())
        return Q4_OK;
    uint32_t err = 0;
    Q4_HIP(hipMemcpy(&err, dec->bar + q4::kBarErr, sizeof(err), hipMemcpyDeviceToHost));
    if (err) {
        // A barrier that gave up leaves arrival words in an unknown state:
        // start over from zero (parity 0, no arrivals).
        Q4_HIP(hipMemset(dec->bar, 0, q4::kBarBytes));
        return q4::fail(Q4_ERR_HIP, "persistent decode: a grid barrier timed out; the step's "
                                    "results are invalid");
    }
    return Q4_OK;
}

// ------------------------------------------------- allocation-free layer
// The intermediates of q4_decode_layer_noalloc live in this array: one copy
// per GPU, held until the process ends.  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol); it
// uses the device address hipGetSymbolAddress returns for the current
// device, looked up once per device and kept in noalloc_ptr.
static __device__ __align__(256) uint8_t scratch[Q4_NOALLOC_SCRATCH_BYTES];

namespace q4 {
namespace {

constexpr int kNoAllocDevices = 64;

// Device address of `scratch` on the current device (nullptr and a status
// on failure), resolved on the first call per device.
q4_status noalloc_ptr(uint8_t **out) {
    static std::mutex mu;
    static uint8_t *ptr[kNoAllocDevices] = {};
    int dev = 0;
    Q4_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= kNoAllocDevices)
        return fail(Q4_ERR_UNSUPPORTED, "q4_decode_layer_noalloc: device index %d >= %d", dev,
                    kNoAllocDevices);
    std::lock_guard<std::mutex> lk(mu);
    if (!ptr[dev]) {
        void *p = nullptr;
        Q4_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (!p || !aligned(p, 256))
            return fail(Q4_ERR_HIP, "q4_decode_layer_noalloc: bad scratch address");
        ptr[dev] = static_cast<uint8_t *>(p);
    }
    *out = ptr[dev];
    return Q4_OK;
}

// Scratch bytes one layer needs: the normed activation (max(d, dff)
// binary16 slots), the fp32 QKV output, the binary16 attention output and
// the binary16 gated MLP activation, each 256-byte aligned.
size_t noalloc_bytes(const Dims &d) {
    return align256(std::max(d.d, d.dff) * 2) + align256(d.nqkv * 4) +
           align256(d.H * d.hd * 2) + align256(d.dff * 2);
}

} // namespace
} // namespace q4

extern "C" q4_status q4_decode_layer_noalloc(const q4_layer *layer, int32_t d_model,
                                             int32_t n_heads, int32_t n_kv_heads,
                                             int32_t head_dim, int32_t d_ff, float eps,
                                             float *h, hipStream_t stream) {
    if (!layer || !h)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_decode_layer_noalloc: null layer or h");
    if (!q4::aligned(h, 16))
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_decode_layer_noalloc: h not 16-byte aligned");
    q4_model_desc m{};
    m.n_layers = 1;
    m.d_model = d_model;
    m.n_heads = n_heads;
    m.n_kv_heads = n_kv_heads;
    m.head_dim = head_dim;
    m.d_ff = d_ff;
    m.eps = eps;
    m.h = h;
    q4::Dims d;
    Q4_CHECK(q4::dims_of(&m, &d));
    Q4_CHECK(q4::check_layer(d, *layer, 0));
    const size_t need = q4::noalloc_bytes(d);
    if (need > (size_t)Q4_NOALLOC_SCRATCH_BYTES)
        return q4::fail(Q4_ERR_UNSUPPORTED,
                        "q4_decode_layer_noalloc: the layer needs %zu scratch bytes, more than "
                        "the %d available",
                        need, Q4_NOALLOC_SCRATCH_BYTES);
    uint8_t *base = nullptr;
    Q4_CHECK(q4::noalloc_ptr(&base));
    // A decoder description on the stack pointing into the scratch array:
    // the same kernels and arguments as q4_decode_layer's (no KV cache).
    q4::Decoder dec;
    dec.desc = m;
    dec.dims = d;
    uint8_t *p = base;
    dec.a16 = reinterpret_cast<uint16_t *>(p);
    p += q4::align256(std::max(d.d, d.dff) * 2);
    dec.qkv = reinterpret_cast<float *>(p);
    p += q4::align256(d.nqkv * 4);
    dec.oin = reinterpret_cast<uint16_t *>(p);
    p += q4::align256(d.H * d.hd * 2);
    dec.mlp = reinterpret_cast<uint16_t *>(p);
    return q4::enqueue_layer(&dec, *layer, -1, stream);
}
