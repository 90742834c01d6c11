// Persistent decode kernel interface (internal).
#pragma once

#include "q4_internal.h"

namespace q4 {

// One layer's four matrices as the persistent kernel reads them from the
// decoder's device-side layer table: qkv, o, gate+up, down.
struct DevLayer {
    const uint8_t *packed[4];
    const uint16_t *scales[4];
};

struct PersistArgs {
    const DevLayer *layers; // device array [n_layers]
    int32_t n_layers;
    float *h;               // fp32 residual [d]
    float *qkv;             // fp32 [(H + 2 Hkv) hd]
    uint16_t *oin;          // binary16 [H hd]
    uint16_t *mlp;          // binary16 [dff]
    uint16_t *norm_out;     // binary16 [d] (second norm, for inspection)
    int32_t d, H, Hkv, hd, dff;
    float eps;
    uint32_t *bar;          // barrier words (kBar* offsets), zeroed at decoder creation
};

// Barrier words of the persistent kernel (uint32 offsets into PersistArgs::bar).
constexpr int kBarParity = 0;       // launch parity bit
constexpr int kBarErr = 1;          // set when a barrier gave up waiting
constexpr int kBarFlags = 64;       // per-workgroup arrival words
constexpr int kMaxPersistentGrid = 4096;
// Bytes of the barrier area: arrival words plus the release word.
constexpr size_t kBarBytes = ((size_t)(kBarFlags + kMaxPersistentGrid + 1) * 4 + 255) & ~(size_t)255;

size_t persistent_lds_bytes(int32_t d, int32_t H, int32_t hd, int32_t dff);
q4_status launch_persistent(const PersistArgs &a, hipStream_t stream);

// Streaming persistent step (producer waves fill an LDS ring): Q4_OK if the
// shapes and the device allow it (every K a multiple of 64, the activation
// plus a ring of at least one unit in LDS, one workgroup per CU resident);
// *nslots gets the ring size.
q4_status stream_supported(int32_t d, int32_t H, int32_t hd, int32_t dff, int *nslots);
q4_status launch_stream(const PersistArgs &a, hipStream_t stream);
// One product (0 QKV, 1 O, 2 gate+up, 3 down) of one layer with the same
// producer/consumer workgroups, as its own launch (no grid barrier).
q4_status launch_stream_product(const PersistArgs &a, int32_t layer, int32_t which,
                                hipStream_t stream);

} // namespace q4
