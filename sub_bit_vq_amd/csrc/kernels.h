// Internal interface between the C ABI (loopvq_host.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/loopvq.h"

namespace lvq {

// Workspace of lvq_decode_attn.  A 256-byte header (a uint32 status word at
// byte 0: kStatus* flags, set by the kernels, read and cleared by
// lvq_decode_status), then a grid of fixed-size blocks, one per (layer, b, h)
// of a call: block i = (layer * B + b) * H + h at kHeaderBytes + i *
// kBlockBytes.  A block holds
//   [0, 8)      the arrival word (uint64): bits 0-31 count the workgroups of
//               the current call that have arrived, bits 32-63 the block's
//               call epoch (calls that merged in it, modulo 2^32 - 1);
//   [256, ...)  kSlots partial slots of (m, l, o[d]), slot s at
//               256 + s * (d + 2) * 8, each value a 64-bit (float bits, tag)
//               pair tagged with epoch + 1 (never 0).
// Every tag written into a block is at most the block's epoch once the call
// has merged, and the next call looks for epoch + 1, so nothing left in a
// block by earlier calls (whatever (layer, b, h, d) they had) matches the
// current call: the grid never moves, and a workspace may serve calls of any
// batch, head count, layer count and head_dim (up to kMaxDecodeDim) without
// being cleared again.
constexpr int kMaxSplits = 64;
constexpr int kSlots = kMaxSplits;
constexpr int kMaxDecodeDim = 128;           // largest head_dim of a decode launch
constexpr uint64_t kHeaderBytes = 256;
constexpr uint64_t kSlotBase = 256;          // byte offset of slot 0 in a block
constexpr uint64_t kBlockBytes = kSlotBase + (uint64_t)kSlots * (kMaxDecodeDim + 2) * 8;
static_assert(kBlockBytes % 256 == 0, "blocks stay 256-byte aligned");
constexpr uint32_t kEpochWrap = 0xffffffffu; // epochs run 0 .. kEpochWrap - 1

// lvq_decode_attn_noalloc's workspace: a static device array holding the
// header and kScratchBlocks blocks (launches that merge may use at most that
// many (layer, b, h) groups)
constexpr uint64_t kScratchBlocks = 256;
constexpr uint64_t kScratchBytes = kHeaderBytes + kScratchBlocks * kBlockBytes;
static_assert(kScratchBlocks == LVQ_NOALLOC_MAX_HEADS && kScratchBytes == LVQ_NOALLOC_SCRATCH_BYTES,
              "the header states the static workspace's size");

// status flags (include/loopvq.h: LVQ_STATUS_*)
constexpr uint32_t kStatusMergeTimeout = 1u;  // a merge gave up waiting; its row is NaN
constexpr uint32_t kStatusValueRange = 2u;    // a value codebook entry outside fp16 range

// Shape of a decode workgroup, shared with the host's split planning: 512
// threads (8 waves); a wave folds 64 / (S/8) tokens per pass and 3 passes per
// batch, so a workgroup steps through its VQ tokens 12288 / S at a time.
constexpr int kDecodeThreads = 512;
constexpr int kDecodeUnroll = 3;
constexpr int decode_batch_tokens(int S) { return kDecodeThreads / 64 * (64 / (S / 8)) * kDecodeUnroll; }

inline uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

// blocks of one layer of a call, and the workspace of a single-layer call
inline uint64_t layer_block_bytes(int64_t B, int64_t H) { return (uint64_t)B * H * kBlockBytes; }
inline uint64_t workspace_bytes(int64_t B, int64_t H) { return kHeaderBytes + layer_block_bytes(B, H); }

// Which (b, h) group and which split role the workgroup with dispatch index p
// takes, in a launch of `total` workgroups that form groups of n consecutive
// logical workgroups.  The hardware deals workgroups to its 8 XCDs in turn
// (XCD p mod 8), so the logical index Lg = (p mod 8) * (total / 8) + p / 8
// puts consecutive logical workgroups (the splits of one group) on one XCD,
// where its L2 serves their shared codebook slices once.  Roles order the
// members of a group by dispatch index: the member dispatched last takes
// role n - 1 (the merger, when the launch merges by window workgroups), so
// every other member of its group was dispatched before it on its own XCD
// or on another one, and a merger never holds a compute unit that one of
// its peers is still waiting for.  A group that lies inside one slab of
// total / 8 logical workgroups keeps role = Lg - first member; one that
// crosses slabs is ranked explicitly.
struct WgRole {
    unsigned group;
    int role;
};
__host__ __device__ inline WgRole decode_role(unsigned p, unsigned total, unsigned n) {
    if (total % 8 != 0) return {p / n, (int)(p % n)};
    const unsigned slab = total / 8;
    const unsigned lg = (p % 8) * slab + p / 8;
    const unsigned g = lg / n, first = g * n, last = first + n - 1;
    if (first / slab == last / slab) return {g, (int)(lg - first)};
    // member lg' of slab sl sits at dispatch index 8 (lg' - sl * slab) + sl:
    // it comes before p = 8 q + s iff (q', sl) < (q, s) lexicographically
    const unsigned q = p / 8, s = p % 8;
    unsigned rank = 0;
    for (unsigned sl = first / slab; sl <= last / slab; ++sl) {
        const unsigned lo = (first > sl * slab ? first : sl * slab) - sl * slab;
        const unsigned hi = (last < sl * slab + slab - 1 ? last : sl * slab + slab - 1) - sl * slab;
        const unsigned lim = sl < s ? q + 1 : q;       // members with q' < lim come first
        if (lim > lo) rank += (lim <= hi ? lim : hi + 1) - lo;
    }
    return {g, (int)rank};
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
                      // slots into w ranges and the others take one VQ chunk
                      // each; 0: each takes a VQ chunk and a range of the
                      // window slots
    int win_per;      // window slots per range: range i is
                      // [i * win_per, (i + 1) * win_per) within [0, W)
    int chunk;        // VQ tokens per chunk (multiple of 64)
    int by_length;    // 1 (one workgroup per (b, h), 2 <= B <= kMaxOrderedBatch,
                      // one layer): workgroups take sequences longest first
                      // in dispatch order
    int cb_bf16;
    int n_layers;     // layers of this launch, 1..kMaxLayersPerLaunch
    int heads_per_wg; // 1, or 2: a workgroup serves query heads 2i, 2i + 1
                      // (one KV head, one layer, window workgroups or
                      // n_split == 1; S = 32, cg = 4, bf16 codebooks)
    const int32_t *ctx_len;     // [B], shared by the layers
    const int32_t *vq_len;      // [B] or null
    int64_t win_bstride;        // elements between sequences of a window buffer
    float scale_log2;           // sm_scale * log2(e)
    // Workspace blocks of the launch's first layer (layer l of the launch,
    // (b, h): block (l * B + b) * H + h from here) and the status word.
    char *blocks;
    uint32_t *status;
    int max_polls;              // bound of a merger's wait, in polls
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
    float *screen;              // null, or [n_tokens][H][S][256]: every screen
                                // value (diagnostic; one tensor, screen path)
};

// Kernel-support predicates (host) and launchers (return the HIP error of the
// launch).
bool decode_supported(int d, int S, int cg, int cb_bf16);
bool encode_supported(int G, int cg, int S, int cb_bf16);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
// device address of the static workspace on the device of `stream` (looked
// up once per device)
hipError_t scratch_address(hipStream_t stream, void **addr);
hipError_t launch_encode(const EncodeArgs &a, hipStream_t stream);

}  // namespace lvq
