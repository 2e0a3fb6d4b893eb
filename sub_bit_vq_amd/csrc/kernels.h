// Internal interface between the C ABI (loopvq_host.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lvq {

// Workspace of lvq_decode_attn: per (b, h), kSlots partial slots of
// (m, l, o[d]), one per split, each value stored as a 64-bit (float bits,
// call tag) pair, then one uint32 arrival word per (b, h): bits 0-7 count the
// workgroups of the current call that have arrived, bits 8-31 count calls.
// Between calls the count is zero (the merging workgroup advances the word).
constexpr int kMaxSplits = 64;
constexpr int kSlots = kMaxSplits;

// Shape of a decode workgroup, shared with the host's split planning: 512
// threads (8 waves); a wave folds 64 / (S/8) tokens per pass and 3 passes per
// batch, so a workgroup steps through its VQ tokens 12288 / S at a time.
constexpr int kDecodeThreads = 512;
constexpr int kDecodeUnroll = 3;
constexpr int decode_batch_tokens(int S) { return kDecodeThreads / 64 * (64 / (S / 8)) * kDecodeUnroll; }

inline uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

inline uint64_t partial_bytes(int64_t B, int64_t H, int64_t d) {
    return align_up((uint64_t)B * H * kSlots * (d + 2) * sizeof(uint64_t), 256);
}
inline uint64_t workspace_bytes(int64_t B, int64_t H, int64_t d) {
    return partial_bytes(B, H, d) + align_up((uint64_t)B * H * sizeof(uint32_t), 256);
}

// Operands of one layer of a decode launch, derived by the host for the
// call's loop step.
struct DecodeLayer {
    const uint16_t *q;          // [B][H][d]
    const uint8_t *k_index;     // [B][Hk][t_max][S] of the step's index group
    const uint8_t *v_index;
    const void *kcb_t;          // codebook slices of step t: [Hk][256][S][cg]
    const void *vcb_t;
    const uint16_t *kwin_t;     // windows of step t: b * win_bstride + [Hk][W][d]
    const uint16_t *vwin_t;
    float *out;                 // [B][H][d]
};
constexpr int kMaxLayersPerLaunch = 16;
constexpr int kMaxOrderedBatch = 256;

struct DecodeArgs {
    int B, H, d, cg, S, n_sink, n_recent;
    int Hk;           // KV heads (caches, codebooks, windows)
    int q_per_kv;     // H / Hk: query head h reads KV head h / q_per_kv
    int64_t t_max;
    int n_split;      // workgroups per (layer, b, h)
    int window_wg;    // w > 0: the last w workgroups of (b, h) split the window
                      // slots into w equal ranges and the others take one VQ
                      // chunk each; 0: each takes a VQ chunk and an equal
                      // share of the window slots
    int chunk;        // VQ tokens per chunk (multiple of 64)
    int by_length;    // 1 (one workgroup per (b, h), 2 <= B <= kMaxOrderedBatch,
                      // one layer): workgroups take sequences longest first
                      // in dispatch order
    int cb_bf16;
    int n_layers;     // layers of this launch, 1..kMaxLayersPerLaunch
    const int32_t *ctx_len;     // [B], shared by the layers
    const int32_t *vq_len;      // [B] or null
    int64_t win_bstride;        // elements between sequences of a window buffer
    float scale_log2;           // sm_scale * log2(e)
    // Workspace of layer l: the single-layer layout at ws + l * ws_stride,
    // partials [B][H][kSlots][d + 2] (value, tag) pairs, then tickets [B][H].
    char *ws;
    uint64_t ws_stride;
    uint64_t ws_tickets;        // byte offset of the tickets in a layer's workspace
    DecodeLayer layer[kMaxLayersPerLaunch];
};

struct EncodeArgs {
    int H, d, Tc, G, cg, S;
    int cb_bf16;
    int n_tensors;              // 1, or 2: a second tensor of the same shape
    const uint16_t *x;
    int64_t sx_tok, sx_head, sx_step;   // element strides of x (and x_b)
    int64_t n_tokens;
    const void *cb;             // [Tc][H][256][S][cg]
    uint8_t *index;             // [B][H][t_max][S]
    const uint16_t *x_b;        // the second tensor (n_tensors == 2): its input,
    const void *cb_b;           // codebook and index cache
    uint8_t *index_b;
    int64_t t_max;
    int64_t seq;
    int64_t first_token;
};

// Kernel-support predicates (host) and launchers (return the HIP error of the
// launch).
bool decode_supported(int d, int S, int cg, int cb_bf16);
bool encode_supported(int G, int cg, int S, int cb_bf16);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_encode(const EncodeArgs &a, hipStream_t stream);

}  // namespace lvq
