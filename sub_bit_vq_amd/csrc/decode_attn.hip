// LoopVQ decode attention for one loop step, gfx950.
//
// LoopVQ project page (mscheong01.github.io/loopvq), "Serving in SGLang --
// Attend from indices": at loop step t the keys and values of the VQ tokens
// are read from shared 8-bit indices through codebook slice t, and the result
// is merged with bf16 attention over the sink and recent tokens.
//
// One launch, n_split * H * B workgroups of 512 threads per layer (a launch
// may hold several layers' buffers: layers are the outermost workgroup
// index).  When the grid fits the chip, workgroup s < n_split - w of (b, h)
// takes VQ tokens [n_s + s*chunk, ...) and the last w split the bf16 window
// slots into w ranges of ceil(W / w) slots; otherwise workgroup s takes a VQ
// chunk and window slots [s*per, (s+1)*per), per = ceil(W / n_split).  The
// host picks n_split, w and chunk.
// With one workgroup per (b, h) over several rounds, workgroups take the
// sequences longest first, in dispatch order.
// A workgroup with VQ tokens stages two tables of (h, t) in LDS, both with one
// 256-byte row per code k (the codebook slice is stored code-major, so row k
// is a contiguous read):
//     score table  [0, 64K):   row k = sm_scale * log2(e) * q_j . Bk_t[k][j]
//                              for j < S, fp32, repeated max(1, 32/S) times
//     value table  [64K, 128K): row k = Bv_t[k][j][0..cg) for j < S (fp16 for
//                              bf16 codebooks, else fp32), repeated to fill
// R = S/8 lanes share a token, each owning 8 sub-vectors.  Lane (token slot
// tk, part r) visits its sub-vectors in an order rotated by tk (and, with a
// replica and read-order choice, offset per lane), so at every step the 32
// lanes of a half-wave read 32 distinct LDS banks: the gathers run without
// bank conflicts.  A gather address is one v_perm_b32 of the code byte and a
// per-lane offset byte: 256*k + offset.
// Every wave keeps its own running max, weight sum and accumulators (online
// softmax, base 2), so the token loop has no barrier; per-token score sums
// use DPP.  Token weights p = 2^(s - m) enter the value sum as fp16
// p * 2^13, and the weight sum adds the same rounded values, so the result is
// an exact weighted average with weights perturbed by at most 2^-11 relative.
// The running max of the VQ tokens lags: it is raised only when a token
// exceeds it by more than 2 (log2).
// Where the R lanes of a token fill whole 4-lane blocks and a gather is 4
// fp16 channels (S = 32, cg = 4: the 0.5-bit head_dim-128 cache), the value
// sums run on the matrix cores: v_mfma_f32_4x4x4_16b_f16 with A = the 4
// gathered rows of a block and B = p' times a one-hot column accumulates
// channel n of all 4 rows in lane n, exactly as p' * v summed in fp32
// (bf16 window values use the fp32 4x4x1 form, so they stay exact).
// Otherwise v_dot2_f32_f16 does them on the vector ALUs.
// Index rows stream from HBM through a three-deep register ring of buffer
// loads; the first batch is issued with the table slices, the second once a
// wave has built its part of the tables (bf16 codebooks: each thread reads the
// 16 bytes of q its part needs, so no wave waits for another's q).  At
// the end the lanes write their (rotated) accumulators to the freed table
// space at their channel positions and the workgroup sums them there.
// Every workgroup but the merger of (b, h) publishes (m, l, o[d]) as 64-bit
// (value, call tag) pairs and leaves.  The merger is the last window
// workgroup when there are any (the member of its group dispatched last, so
// its peers were dispatched before it), else the last to take an arrival
// ticket once its tokens are done (the round trip overlaps its own
// reduction).  It polls the others' pairs until every tag is the current
// call's, merges (log-sum-exp, slots in ascending order, its own from
// registers, so the result does not depend on which workgroup merges) into
// out and advances the block's epoch to the next call.  Everything crosses
// workgroups through agent-scope atomics (no L2 writeback or invalidation);
// each pair is one 64-bit access, so no store needs a completion wait.
#include "kernels.h"

#include <math.h>

#include <mutex>
#include <type_traits>

// Workspace of lvq_decode_attn_noalloc: a file-scope device array (zero at
// load, one copy per device, held until the process ends).  Host code never
// passes its name to a kernel (on the host it is only a stand-in for the
// symbol); it passes the device address that hipGetSymbolAddress returns for
// the device the call runs on (lvq::scratch_address).
static __device__ __align__(256) unsigned char scratch[lvq::kScratchBytes];

namespace lvq {
namespace {

constexpr int kThreads = kDecodeThreads;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = kDecodeUnroll;         // token passes per batch
constexpr float kPScale = 8192.f;              // p' = p * 2^13 (normal in fp16 down to p ~ 7e-9)
constexpr float kMaxSlack = 2.f;               // a VQ token may exceed the running max by this
                                               // (log2) before it is raised: p' <= 2^15
constexpr int kLdsLimit = 160 * 1024;
constexpr int kMergeChunk = 16;                // partial slots loaded per poll
constexpr int kVTab = 65536;                   // LDS byte offset of the value table
constexpr int kBufferWord3 = 0x00020000;       // raw buffer resource, gfx9 family
constexpr int kTabBytes = 131072;              // both tables

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));

// 2^x by the hardware instruction (results below 2^-126 flush to zero,
// which no weight here can tell apart from zero)
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <int S, int CG, typename CB>
struct Shape {
    static constexpr int D = S * CG;
    static constexpr int R = S / 8;                   // lanes per token
    static constexpr int TPW = 64 / R;                // tokens per wave pass
    static constexpr int CL = 8 * CG;                 // output channels per lane
    static constexpr bool kF16V = std::is_same<CB, uint16_t>::value;
    static constexpr int VB = kF16V ? 2 : 4;          // bytes per value-table element
    static constexpr int EB = CG * VB;                // bytes per value-table entry
    static constexpr int RB = EB <= 4 ? EB : 8;       // bytes per value read (b32 or b64)
    static constexpr int NRD = EB / RB;               // reads per value gather
    static constexpr int CPR = RB / VB;               // channels per read
    // score-table replicas per 64-float row: enough for the lanes of a
    // half-wave to read distinct banks (a row is 256 bytes either way)
    static constexpr int KCOP = S >= 32 ? 1 : 32 / S;
    static constexpr int VCOP = 256 / (S * EB);       // value-table replicas per row
    static constexpr int SRCB = CG * (int)sizeof(CB); // codebook bytes per entry
    static constexpr int UNIT = SRCB > 16 ? SRCB : 16;   // staging load bytes
    static constexpr int EPU = UNIT / SRCB;           // entries per staging unit
    static constexpr int UPT = S * 256 / EPU / kThreads;   // staging units per thread
    static constexpr int NACC = 8 * CG;               // accumulators per lane
    // Value sums on the matrix cores: the 4 lanes of a 4x4x4 MFMA block are
    // parts of one token (R a multiple of 4) and a gather is 4 fp16 channels.
    static constexpr bool kMfma = kF16V && EB == 8 && R % 4 == 0;
    static constexpr int G = kThreads / D;            // reduction groups per channel
    // Epilogue dump of the lane accumulators (rows = token slots of the
    // workgroup).  For head_dim 64 and 128, rows are padded by 16 bytes, so
    // that 16 consecutive rows read at one 16-byte offset hit distinct banks,
    // and each thread sums 4 positions of every SS-th row.
    static constexpr bool kQuadRed = D == 64 || D == 128;
    // Token slots tk and tk + TPW/2 (lanes 32 apart) fold in registers before
    // the dump when their accumulators hold the same channels: with MFMA value
    // sums, and with the plain ones at R <= 2 (the same rotation, and the
    // same order of a sub-vector's value reads: sw below)
    static constexpr bool kFold =
        kMfma || (kQuadRed && R <= 2 && (TPW / 2) % (8 * VCOP) == 0 && ((TPW / 2) / (8 * VCOP)) % NRD == 0);
    // dump rows: one per token slot, or per pair of slots when they fold
    static constexpr int NR = kFold ? kWaves * TPW / 2 : kWaves * TPW;
    static constexpr int RS = kQuadRed ? D * 4 + 16 : D * 4;   // row stride, bytes
    static constexpr int kDumpBytes = NR * RS;
    static constexpr int kBase = kDumpBytes > kTabBytes ? kDumpBytes : kTabBytes;
    // q (up to two heads), wave stats, reduction partials, arrival words
    static constexpr int kExtra = 4 * (2 * D + 4 * kWaves + kThreads) + 16;
    static constexpr int kLds = kBase + kExtra;
    static_assert(S >= 8 && S <= 64 && (S & (S - 1)) == 0, "8 sub-vectors per lane");
    static_assert(S * EB <= 256, "a value-table row holds every sub-vector");
    static_assert(UPT * EPU * kThreads == S * 256, "staging tiles the tables");
    static_assert(kQuadRed || kWaves * TPW * D * 4 <= kTabBytes, "the lane dump fits the tables");
    static_assert(kThreads % D == 0 && TPW % G == 0, "reduction tiling");
    static_assert(kWaves * TPW * kUnroll == decode_batch_tokens(S), "the host plans with this batch");
};

struct Windows {
    int L, n_s, n_v;
};

// Windows of a sequence from its raw length and VQ count (vq < 0: exact
// windows), clamped to the documented preconditions.
__device__ __forceinline__ Windows seq_windows(int Lraw, int vqraw, int64_t t_max, int n_sink,
                                               int n_recent) {
    const int L = max(0, (int)min((int64_t)Lraw, t_max));
    const int n_s = min(L, n_sink);
    const int n_v = vqraw >= 0 ? max(0, min(vqraw, L - n_s)) : max(0, L - n_sink - n_recent);
    return {L, n_s, n_v};
}

// Does window slot `slot` hold a token of the current sink/recent windows?
// Recent token p sits in slot n_sink + ((p - n_sink) mod n_recent); the slot
// holds the newest such p below L.
__device__ __forceinline__ bool slot_valid(int slot, const Windows &w, int n_sink, int n_recent) {
    if (slot < n_sink) return slot < w.n_s;
    if (w.L <= n_sink) return false;
    const int r = slot - n_sink;
    const int A = w.L - 1 - n_sink;
    if (r > A) return false;
    const int pos = n_sink + r + n_recent * ((A - r) / n_recent);
    return pos >= w.n_s + w.n_v;
}

// DPP lane permutations (VALU only): quad_perm xor 1, xor 2, row_ror 4, 8,
// row_half_mirror
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kXor1 = 0xB1, kXor2 = 0x4E, kRor4 = 0x124, kRor8 = 0x128, kHalfMirror = 0x141;

__device__ __forceinline__ float lane_f(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// After pair16(x, a, b), {a, b} of every lane hold x of that lane and of lane
// ^ 16 (a + b is then their sum in both)
__device__ __forceinline__ void pair16(float x, float &a, float &b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}

// sum over the R consecutive lanes of a token
template <int R>
__device__ __forceinline__ float token_sum(float v) {
    if constexpr (R >= 2) v += dppf<kXor1>(v);
    if constexpr (R >= 4) v += dppf<kXor2>(v);
    if constexpr (R >= 8) v += dppf<kHalfMirror>(v);
    return v;
}

// maximum / sum over the 16 lanes of a row, in every lane of it
__device__ __forceinline__ float row_max(float v) {
    v = fmaxf(v, dppf<kXor1>(v));
    v = fmaxf(v, dppf<kXor2>(v));
    v = fmaxf(v, dppf<kRor4>(v));
    return fmaxf(v, dppf<kRor8>(v));
}
__device__ __forceinline__ float row_sum(float v) {
    v += dppf<kXor1>(v);
    v += dppf<kXor2>(v);
    v += dppf<kRor4>(v);
    return v + dppf<kRor8>(v);
}

// wave-uniform maximum / sum
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dppf<kXor1>(v));
    v = fmaxf(v, dppf<kXor2>(v));
    v = fmaxf(v, dppf<kRor4>(v));
    v = fmaxf(v, dppf<kRor8>(v));
    return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
    v += dppf<kXor1>(v);
    v += dppf<kXor2>(v);
    v += dppf<kRor4>(v);
    v += dppf<kRor8>(v);
    return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

// one 64-bit (value, tag) pair of a published partial
__device__ __forceinline__ void publish(uint64_t *p, float v, uint32_t tag) {
    __hip_atomic_store(p, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// bytes of the 64-bit value (hi:lo) picked by the four selector bytes of sel
// (0-3: bytes of lo, 4-7: bytes of hi, 12: zero)
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// The larger magnitude of each 16-bit half: a running maximum over bf16
// pairs.  value_out_of_fp16 then says whether either half is outside fp16's
// finite range (|v| >= 2^16, or not finite; no bf16 value lies in
// (65280, 65536)).
__device__ __forceinline__ uint32_t max_halves(uint32_t mx, uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(ushort2_t, mx),
                                                                  __builtin_bit_cast(ushort2_t, w & 0x7fff7fffu)));
}
__device__ __forceinline__ bool value_out_of_fp16(uint32_t mx) {
    return (mx & 0xffffu) >= 0x4780u || (mx >> 16) >= 0x4780u;
}

// Per-lane gather constants.  At step i (0..7) lane (tk, r) handles
// sub-vector j_i = 8r + ((i + rot) mod 8).  Its score read is at byte
// 256k + offK_i, offK_i = 4 (S*copyK + j_i); its value reads at
// 64K + 256k + offV_i (xor 8h for the h-th 8-byte read of an entry).  The
// offsets sit one per byte in offK / offV words (offV words also carry the
// 64K bit), so that one v_perm_b32 of (offset word, index word) is the address.
template <int S, int CG, typename CB>
struct Lanes {
    using Sh = Shape<S, CG, CB>;
    uint32_t rotA, rotB;         // selectors: index bytes in step order
    uint32_t offK[2], offV[4];
    uint32_t bmask0, bmask1;     // MFMA B operand: the lane's column in a 4-lane block
    int rot, sw, r;

    __device__ __forceinline__ void init(int lane) {
        const int tk = lane / Sh::R;
        r = lane % Sh::R;
        rot = (tk + 4 * (r >> 2)) & 7;
        const int n = r & 3;
        bmask0 = n == 0 ? 0x0000ffffu : n == 1 ? 0xffff0000u : 0u;
        bmask1 = n == 2 ? 0x0000ffffu : n == 3 ? 0xffff0000u : 0u;
        const int copyK = (tk >> 3) % Sh::KCOP;
        const int copyV = (tk >> 3) % Sh::VCOP;
        sw = (tk / (8 * Sh::VCOP)) % Sh::NRD;
        rotA = rotB = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            rotA |= (uint32_t)((rot + b) & 7) << (8 * b);
            rotB |= (uint32_t)((rot + 4 + b) & 7) << (8 * b);
        }
        offK[0] = offK[1] = 0;
#pragma unroll
        for (int m = 0; m < 4; ++m) offV[m] = 1u << 16;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int j = 8 * r + ((i + rot) & 7);
            offK[i >> 2] |= (uint32_t)(4 * (S * copyK + j)) << (8 * (i & 3));
            const uint32_t ov = Sh::EB <= 4 ? 4u * (S * copyV + j)
                                            : 8u * (Sh::NRD * (S * copyV + j) + sw);
            offV[i >> 1] |= ov << (8 * (i & 1));
        }
    }
    // channel of read h of step i (output position of its first element)
    __device__ __forceinline__ int channel(int i, int h) const {
        return (8 * r + ((i + rot) & 7)) * CG + Sh::CPR * (h ^ sw);
    }
};

// perm selectors: byte 0 = offset byte, byte 1 = index byte, then zero
// (score) or the 64K byte of the offset word and zero (value)
__device__ __forceinline__ constexpr uint32_t sel_k(int i) {
    return 0x0c0c0000u | ((uint32_t)(i & 3) << 8) | (uint32_t)(4 + (i & 3));
}
__device__ __forceinline__ constexpr uint32_t sel_v(int i) {
    return 0x0c060000u | ((uint32_t)(i & 3) << 8) | (uint32_t)(4 + (i & 1));
}

// Per-wave online-softmax state: running max m (base 2), weight sum l (scaled
// by 2^13; every lane of a token adds its weight, so the wave sum counts each
// token R times) and accumulators.
template <int NACC>
struct Online {
    float m = -INFINITY;
    float l = 0.f;
    float acc[NACC];

    __device__ __forceinline__ void init() {
#pragma unroll
        for (int i = 0; i < NACC; ++i) acc[i] = 0.f;
    }
    // raise the running max to at least `mx` (wave-uniform)
    __device__ __forceinline__ void raise(float mx) {
        if (mx > m) {
            // a real (wave-uniform) branch: the rescale is rare after the first
            // batches, and the compiler would otherwise execute it every time
            __asm__ volatile("");
            const float sc = ex2(m - mx);     // 0 when m = -inf
            l *= sc;
#pragma unroll
            for (int i = 0; i < NACC; ++i) acc[i] *= sc;
            m = mx;
        }
    }
};

// ---------------------------------------------------------------------------
// Table staging for (h, loop step t), in two phases so that the loads can be
// issued before q is known: load() reads the K and V slices ([256][S][cg],
// code-major) into registers, finish() writes both tables into LDS.
// ---------------------------------------------------------------------------
template <int S, int CG, typename CB>
struct Stage {
    using Sh = Shape<S, CG, CB>;
    static constexpr int UW = Sh::UNIT / 4;           // 32-bit words per unit
    uint32_t kw[Sh::UPT][UW], vw[Sh::UPT][UW];

    // kr, vr: the slices as buffer resources (a zero-length one reads zeros
    // and moves no data: workgroups without VQ tokens issue the same loads)
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr) {
        const uint32_t off = threadIdx.x * Sh::UNIT;
#pragma unroll
        for (int u = 0; u < Sh::UPT; ++u) {
            const uint32_t so = (uint32_t)(u * kThreads * Sh::UNIT);
#pragma unroll
            for (int w = 0; w < UW; w += 4) {
                const uint4 x = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, off + 4 * w, so, 0));
                const uint4 y = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vr, off + 4 * w, so, 0));
                kw[u][w] = x.x; kw[u][w + 1] = x.y; kw[u][w + 2] = x.z; kw[u][w + 3] = x.w;
                vw[u][w] = y.x; vw[u][w + 1] = y.y; vw[u][w + 2] = y.z; vw[u][w + 3] = y.w;
            }
        }
    }

    __device__ __forceinline__ float elem(const uint32_t *w, int i) const {
        if constexpr (Sh::kF16V) return (i & 1) ? bf16hi(w[i >> 1]) : bf16lo(w[i >> 1]);
        else return __uint_as_float(w[i]);
    }

    // qs: the scaled query (fp32, LDS; used with fp32 codebooks); qw: with
    // bf16 codebooks, this thread's raw bf16 query words, two channels a word:
    // the EPU entries of every unit it stages are sub-vectors j0 .. j0 + EPU - 1
    // with the same j0 = (tid * EPU) mod S, so one 16-byte piece of q serves
    // them all.  Returns whether a bf16 value entry of the units in `check`
    // (bit u: unit u) falls outside fp16's range (value_out_of_fp16).
    // NH query heads (consecutive, one KV head): head hh's score table
    // takes the replica slots KCOP*hh .. of every row (NH = 2: S = 32, one
    // replica, so the second head's scores fill the upper half of the row).
    template <int NH>
    __device__ __forceinline__ bool finish(const float *qs, const uint32_t (*qw)[4], float scale,
                                           unsigned char *smem, uint32_t check) const {
        static_assert(NH == 1 || Sh::kF16V, "head pairs: bf16 codebooks");
        const int tid = threadIdx.x;
        float *lutk = reinterpret_cast<float *>(smem);
        uint32_t mx = 0;
#pragma unroll
        for (int u = 0; u < Sh::UPT; ++u) {
            const int e0 = (tid + u * kThreads) * Sh::EPU;   // first entry of the unit
            const int k = e0 / S, j0 = e0 % S;
#pragma unroll
          for (int hh = 0; hh < NH; ++hh) {
            float accs[Sh::EPU];
#pragma unroll
            for (int e = 0; e < Sh::EPU; ++e) {
                const int j = j0 + e;
                float acc = 0.f;
                if constexpr (Sh::kF16V) {
                    // bf16 pairs: exact products, then one scaling
                    constexpr int WPE = CG / 2;
#pragma unroll
                    for (int m = 0; m < WPE; ++m)
                        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qw[hh][e * WPE + m]),
                                                              __builtin_bit_cast(bf16x2_t, kw[u][e * WPE + m]),
                                                              acc, false);
                    acc *= scale;
                } else {
#pragma unroll
                    for (int c = 0; c < CG; ++c) acc += qs[j * CG + c] * elem(kw[u], e * CG + c);
                }
                accs[e] = acc;
            }
            // a unit's entries are adjacent in the row: written together
#pragma unroll
            for (int cp = 0; cp < Sh::KCOP; ++cp) {
                float *row = lutk + k * 64 + S * (Sh::KCOP * hh + cp) + j0;
                if constexpr (Sh::EPU % 4 == 0) {
#pragma unroll
                    for (int e = 0; e < Sh::EPU; e += 4)
                        *reinterpret_cast<float4 *>(row + e) = make_float4(accs[e], accs[e + 1], accs[e + 2], accs[e + 3]);
                } else if constexpr (Sh::EPU % 2 == 0) {
#pragma unroll
                    for (int e = 0; e < Sh::EPU; e += 2)
                        *reinterpret_cast<float2 *>(row + e) = make_float2(accs[e], accs[e + 1]);
                } else {
                    row[0] = accs[0];
                }
            }
          }
            // value entries of the unit, converted, into every replica of row k
            uint32_t o[UW];
#pragma unroll
            for (int w = 0; w < UW; ++w) {
                if constexpr (Sh::kF16V) {
                    // bf16 -> fp16 is exact within fp16's range, so the
                    // rounding mode of the packed conversion does not matter
                    o[w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(bf16lo(vw[u][w]), bf16hi(vw[u][w])));
                } else {
                    o[w] = vw[u][w];
                }
            }
            if constexpr (Sh::kF16V) {
                if ((check >> u) & 1u) {                  // wave-uniform
#pragma unroll
                    for (int w = 0; w < UW; ++w) mx = max_halves(mx, vw[u][w]);
                }
            }
#pragma unroll
            for (int cp = 0; cp < Sh::VCOP; ++cp) {
                uint4 *dst = reinterpret_cast<uint4 *>(smem + kVTab + k * 256 + (S * cp + j0) * Sh::EB);
#pragma unroll
                for (int w = 0; w < UW; w += 4) dst[w / 4] = make_uint4(o[w], o[w + 1], o[w + 2], o[w + 3]);
            }
        }
        return value_out_of_fp16(mx);
    }
};

// ---------------------------------------------------------------------------
// Dense bf16 window slots [s0, s1): R lanes per slot.  The key dot product
// uses the lane's contiguous CL channels; the value row is read in the
// lane's gather order so that it lands on the same accumulators.
// ---------------------------------------------------------------------------
template <int S, int CG, typename CB>
struct WindowPass {
    using Sh = Shape<S, CG, CB>;
    static constexpr int CL = Sh::CL, NRD = Sh::NRD, CPR = Sh::CPR;
    uint32_t k[CL / 2];
    uint32_t v[8 * NRD][CPR / 2];
    int slot;
    bool in;

    // kw, vw: the [W][d] window rows of (b, t, h).  Rows are read only for
    // slots of this workgroup (host-known, so the loads need not wait for the
    // context length); whether a slot holds a token is decided at fold time.
    __device__ __forceinline__ void load(const uint16_t *kw, const uint16_t *vw, int slot_, int s1,
                                         const Lanes<S, CG, CB> &ln) {
        constexpr int D = Sh::D;
        slot = slot_;
        in = slot < s1;
        if (!in) {
#pragma unroll
            for (int i = 0; i < CL / 2; ++i) k[i] = 0u;
#pragma unroll
            for (int i = 0; i < 8 * NRD; ++i)
#pragma unroll
                for (int e = 0; e < CPR / 2; ++e) v[i][e] = 0u;
            return;
        }
        const uint4 *kp = reinterpret_cast<const uint4 *>(kw + (size_t)slot * D + ln.r * CL);
#pragma unroll
        for (int i = 0; i < CL / 8; ++i) {
            const uint4 kk = kp[i];
            k[4 * i] = kk.x; k[4 * i + 1] = kk.y; k[4 * i + 2] = kk.z; k[4 * i + 3] = kk.w;
        }
        const uint16_t *vrow = vw + (size_t)slot * D;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
            for (int h = 0; h < NRD; ++h) {
                const uint16_t *p = vrow + ln.channel(i, h);
                if constexpr (CPR == 4) {
                    const uint2 t = *reinterpret_cast<const uint2 *>(p);
                    v[i * NRD + h][0] = t.x;
                    v[i * NRD + h][1] = t.y;
                } else {
                    v[i * NRD + h][0] = *reinterpret_cast<const uint32_t *>(p);
                }
            }
        }
    }

    template <typename OnlineT>
    __device__ __forceinline__ void fold(const float *qs, OnlineT &st, int r, const Windows &w,
                                         int n_sink, int n_recent) {
        constexpr int R = Sh::R;
        const bool ok = in && slot_valid(slot, w, n_sink, n_recent);
        float dot = 0.f;
        if (ok) {
#pragma unroll
            for (int i = 0; i < CL / 2; ++i) {
                dot += qs[r * CL + 2 * i] * bf16lo(k[i]);
                dot += qs[r * CL + 2 * i + 1] * bf16hi(k[i]);
            }
        }
        dot = token_sum<R>(dot);
        const float s = ok ? dot : -INFINITY;
        const float mx = wave_max(s);
        if (mx == -INFINITY) return;              // wave-uniform
        st.raise(mx);
        const float p = ok ? ex2(s - st.m) * kPScale : 0.f;
        st.l += p;
        if constexpr (Sh::kMfma) {
            // column c of the block gets p; rows are the 4 lanes' values
            const int n = r & 3;
            float bc[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) bc[c] = n == c ? p : 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float4_t d = {st.acc[4 * i], st.acc[4 * i + 1], st.acc[4 * i + 2], st.acc[4 * i + 3]};
                d = __builtin_amdgcn_mfma_f32_4x4x1f32(bf16lo(v[i][0]), bc[0], d, 0, 0, 0);
                d = __builtin_amdgcn_mfma_f32_4x4x1f32(bf16hi(v[i][0]), bc[1], d, 0, 0, 0);
                d = __builtin_amdgcn_mfma_f32_4x4x1f32(bf16lo(v[i][1]), bc[2], d, 0, 0, 0);
                d = __builtin_amdgcn_mfma_f32_4x4x1f32(bf16hi(v[i][1]), bc[3], d, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) st.acc[4 * i + e] = d[e];
            }
            return;
        }
#pragma unroll
        for (int q = 0; q < 8 * NRD; ++q) {
#pragma unroll
            for (int e = 0; e < CPR / 2; ++e) {
                st.acc[q * CPR + 2 * e] += p * bf16lo(v[q][e]);
                st.acc[q * CPR + 2 * e + 1] += p * bf16hi(v[q][e]);
            }
        }
    }

    // The same slot for two query heads (q of head hh at qs + hh * D): the
    // rows are read once, each head scores them and takes the values with its
    // own weight.
    template <typename OnlineT>
    __device__ __forceinline__ void fold_pair(const float *qs, OnlineT *sts, int r, const Windows &w,
                                              int n_sink, int n_recent) {
        static_assert(Sh::kMfma, "head pairs: the MFMA shape");
        constexpr int R = Sh::R, D = Sh::D;
        const bool ok = in && slot_valid(slot, w, n_sink, n_recent);
        const int n = r & 3;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            OnlineT &st = sts[hh];
            const float *qh = qs + hh * D;
            float dot = 0.f;
            if (ok) {
#pragma unroll
                for (int i = 0; i < CL / 2; ++i) {
                    dot += qh[r * CL + 2 * i] * bf16lo(k[i]);
                    dot += qh[r * CL + 2 * i + 1] * bf16hi(k[i]);
                }
            }
            dot = token_sum<R>(dot);
            const float s = ok ? dot : -INFINITY;
            const float mx = wave_max(s);
            if (mx == -INFINITY) return;          // wave-uniform, the same for both heads
            st.raise(mx);
            const float p = ok ? ex2(s - st.m) * kPScale : 0.f;
            st.l += p;
            float bc[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) bc[c] = n == c ? p : 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float4_t d = {st.acc[4 * i], st.acc[4 * i + 1], st.acc[4 * i + 2], st.acc[4 * i + 3]};
                d = __builtin_amdgcn_mfma_f32_4x4x1f32(bf16lo(v[i][0]), bc[0], d, 0, 0, 0);
                d = __builtin_amdgcn_mfma_f32_4x4x1f32(bf16hi(v[i][0]), bc[1], d, 0, 0, 0);
                d = __builtin_amdgcn_mfma_f32_4x4x1f32(bf16lo(v[i][1]), bc[2], d, 0, 0, 0);
                d = __builtin_amdgcn_mfma_f32_4x4x1f32(bf16hi(v[i][1]), bc[3], d, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) st.acc[4 * i + e] = d[e];
            }
        }
    }
};

// ---------------------------------------------------------------------------
// VQ tokens: a batch is kUnroll wave passes of index rows (8 bytes of the K
// row and 8 of the V row per lane); batches rotate through a 3-deep ring.
// ---------------------------------------------------------------------------
struct Batch {
    uint2 k[kUnroll], v[kUnroll];
};

// The index rows of one (b, h) as buffer resources that end at the last row
// the workgroup may use: a read past it returns zeros (code 0, masked later)
// without touching memory, so loads need neither clamps nor 64-bit address
// arithmetic, every batch issues the same number of loads, and the ring's
// run-ahead past the range costs no HBM traffic.
struct IndexRows {
    __amdgpu_buffer_rsrc_t k, v;
    uint32_t lane;                              // byte offset of the lane: tk*S + 8r

    __device__ __forceinline__ void init(const uint8_t *kbase, const uint8_t *vbase, int rows,
                                         uint32_t lane_off, int S) {
        k = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(kbase), (short)0, rows * S,
                                              kBufferWord3);
        v = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(vbase), (short)0, rows * S,
                                              kBufferWord3);
        lane = lane_off;
    }
};

// Index rows are read once per call: the loads carry the non-temporal hint,
// so that the stream does not push the kernel's code and the codebook slices
// out of L2 (measured: 16.5 -> 15.9 us at 32K, 0.5 bit).
constexpr int kStreamPolicy = 2;                   // cache policy bits: nt

template <int S, int CG, typename CB>
__device__ __forceinline__ void load_batch(const IndexRows &ir, int base, Batch &bt) {
    using Sh = Shape<S, CG, CB>;
    constexpr int STEP = kWaves * Sh::TPW;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const uint32_t off = ir.lane + (uint32_t)(base + u * STEP) * S;
        bt.k[u] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(ir.k, off, 0, kStreamPolicy));
        bt.v[u] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(ir.v, off, 0, kStreamPolicy));
    }
}

template <int S, int CG, typename CB, typename OnlineT>
__device__ __forceinline__ void fold_batch(const Batch &bt, int base, int t1,
                                           const unsigned char *smem,
                                           const Lanes<S, CG, CB> &ln, OnlineT &st) {
    using Sh = Shape<S, CG, CB>;
    constexpr int R = Sh::R, STEP = kWaves * Sh::TPW, NRD = Sh::NRD, CPR = Sh::CPR;
    const int tk = (threadIdx.x & 63) / R;
    float s[kUnroll];
    bool ok[kUnroll];
    float mx = -INFINITY;
    // all score gathers of the batch go out before any is summed (the LDS
    // latency then overlaps), and each token's 8 values are summed as a tree
    float g[kUnroll][8];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const uint32_t w0 = perm(bt.k[u].y, bt.k[u].x, ln.rotA);   // index bytes in step order
        const uint32_t w1 = perm(bt.k[u].y, bt.k[u].x, ln.rotB);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            g[u][i] = *reinterpret_cast<const float *>(smem + perm(ln.offK[i >> 2], i < 4 ? w0 : w1, sel_k(i)));
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        ok[u] = base + u * STEP + tk < t1;
        float acc = ((g[u][0] + g[u][1]) + (g[u][2] + g[u][3])) + ((g[u][4] + g[u][5]) + (g[u][6] + g[u][7]));
        acc = token_sum<R>(acc);
        s[u] = ok[u] ? acc : -INFINITY;
        mx = fmaxf(mx, s[u]);
    }
    // The running max is raised only when a token of the batch exceeds it by
    // more than kMaxSlack (rare after the first batch): the weights of the
    // others stay exact relative to it, and p' = 2^(s - m) * 2^13 <= 2^15 fits
    // fp16.  A ballot replaces a wave-wide max reduction per batch.
    if (__ballot(mx > st.m + kMaxSlack) != 0) st.raise(wave_max(mx));
    if constexpr (Sh::kMfma) {
        // value gathers of pass u + 1 go out before the MFMAs of pass u
        uint2 av[2][8];
        auto gather = [&](int u, uint2 *dst) {
            const uint32_t w0 = perm(bt.v[u].y, bt.v[u].x, ln.rotA);
            const uint32_t w1 = perm(bt.v[u].y, bt.v[u].x, ln.rotB);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                dst[i] = *reinterpret_cast<const uint2 *>(smem + perm(ln.offV[i >> 1], i < 4 ? w0 : w1, sel_v(i)));
        };
        gather(0, av[0]);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (u + 1 < kUnroll) gather(u + 1, av[(u + 1) & 1]);
            // tokens past the range take weight 0 (out-of-range rows read code 0)
            const _Float16 ph = (_Float16)(ok[u] ? ex2(s[u] - st.m) * kPScale : 0.f);
            st.l += (float)ph;
            const uint32_t ph2 = (uint32_t)__builtin_bit_cast(uint16_t, ph) * 0x00010001u;
            const half4_t bop = __builtin_bit_cast(half4_t, make_uint2(ph2 & ln.bmask0, ph2 & ln.bmask1));
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float4_t d = {st.acc[4 * i], st.acc[4 * i + 1], st.acc[4 * i + 2], st.acc[4 * i + 3]};
                d = __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(half4_t, av[u & 1][i]), bop, d, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) st.acc[4 * i + e] = d[e];
            }
        }
        return;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        // tokens past the range take weight 0 (out-of-range rows read code 0)
        const uint32_t w0 = perm(bt.v[u].y, bt.v[u].x, ln.rotA);
        const uint32_t w1 = perm(bt.v[u].y, bt.v[u].x, ln.rotB);
        if constexpr (Sh::kMfma) {
            // handled below, one pass ahead
        } else if constexpr (Sh::kF16V) {
            const _Float16 ph = (_Float16)(ok[u] ? ex2(s[u] - st.m) * kPScale : 0.f);
            st.l += (float)ph;
            const half2_t plo = {ph, (_Float16)0.f};
            const half2_t phi = {(_Float16)0.f, ph};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t ad = perm(ln.offV[i >> 1], i < 4 ? w0 : w1, sel_v(i));
#pragma unroll
                for (int h = 0; h < NRD; ++h) {
                    float *acc = st.acc + (i * NRD + h) * CPR;
                    if constexpr (CPR == 4) {
                        const uint2 e = *reinterpret_cast<const uint2 *>(smem + (ad ^ (8u * h)));
                        const half2_t e0 = __builtin_bit_cast(half2_t, e.x);
                        const half2_t e1 = __builtin_bit_cast(half2_t, e.y);
                        acc[0] = __builtin_amdgcn_fdot2(e0, plo, acc[0], false);
                        acc[1] = __builtin_amdgcn_fdot2(e0, phi, acc[1], false);
                        acc[2] = __builtin_amdgcn_fdot2(e1, plo, acc[2], false);
                        acc[3] = __builtin_amdgcn_fdot2(e1, phi, acc[3], false);
                    } else {
                        const half2_t e0 =
                            __builtin_bit_cast(half2_t, *reinterpret_cast<const uint32_t *>(smem + ad));
                        acc[0] = __builtin_amdgcn_fdot2(e0, plo, acc[0], false);
                        acc[1] = __builtin_amdgcn_fdot2(e0, phi, acc[1], false);
                    }
                }
            }
        } else {
            const float p = ok[u] ? ex2(s[u] - st.m) * kPScale : 0.f;
            st.l += p;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t ad = perm(ln.offV[i >> 1], i < 4 ? w0 : w1, sel_v(i));
#pragma unroll
                for (int h = 0; h < NRD; ++h) {
                    const float2 e = *reinterpret_cast<const float2 *>(smem + (ad ^ (8u * h)));
                    float *acc = st.acc + (i * NRD + h) * CPR;
                    acc[0] += p * e.x;
                    acc[1] += p * e.y;
                }
            }
        }
    }
}

// A batch for two query heads of one KV head (kModePair): every index row is
// read and decoded once; each lane's score gathers for the second head use
// the same addresses 4S bytes further (the upper half of the table row), and
// the value gathers are shared, each head summing them with its own weights.
template <int S, int CG, typename CB, typename OnlineT>
__device__ __forceinline__ void fold_pair(const Batch &bt, int base, int t1,
                                          const unsigned char *smem,
                                          const Lanes<S, CG, CB> &ln, OnlineT *sts) {
    using Sh = Shape<S, CG, CB>;
    static_assert(Sh::kMfma && Sh::KCOP == 1, "head pairs: the MFMA shape");
    constexpr int R = Sh::R, STEP = kWaves * Sh::TPW;
    constexpr uint32_t kSecond = 4 * S;               // second head's scores in a row
    const int tk = (threadIdx.x & 63) / R;
    float s[2][kUnroll];
    bool ok[kUnroll];
    float mx[2] = {-INFINITY, -INFINITY};
    float g[kUnroll][2][8];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const uint32_t w0 = perm(bt.k[u].y, bt.k[u].x, ln.rotA);   // index bytes in step order
        const uint32_t w1 = perm(bt.k[u].y, bt.k[u].x, ln.rotB);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t ad = perm(ln.offK[i >> 2], i < 4 ? w0 : w1, sel_k(i));
            g[u][0][i] = *reinterpret_cast<const float *>(smem + ad);
            g[u][1][i] = *reinterpret_cast<const float *>(smem + ad + kSecond);
        }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        ok[u] = base + u * STEP + tk < t1;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const float *gg = g[u][hh];
            float acc = ((gg[0] + gg[1]) + (gg[2] + gg[3])) + ((gg[4] + gg[5]) + (gg[6] + gg[7]));
            acc = token_sum<R>(acc);
            s[hh][u] = ok[u] ? acc : -INFINITY;
            mx[hh] = fmaxf(mx[hh], s[hh][u]);
        }
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
        if (__ballot(mx[hh] > sts[hh].m + kMaxSlack) != 0) sts[hh].raise(wave_max(mx[hh]));
    uint2 av[2][8];
    auto gather = [&](int u, uint2 *dst) {
        const uint32_t w0 = perm(bt.v[u].y, bt.v[u].x, ln.rotA);
        const uint32_t w1 = perm(bt.v[u].y, bt.v[u].x, ln.rotB);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            dst[i] = *reinterpret_cast<const uint2 *>(smem + perm(ln.offV[i >> 1], i < 4 ? w0 : w1, sel_v(i)));
    };
    gather(0, av[0]);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        if (u + 1 < kUnroll) gather(u + 1, av[(u + 1) & 1]);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            OnlineT &st = sts[hh];
            // tokens past the range take weight 0 (out-of-range rows read code 0)
            const _Float16 ph = (_Float16)(ok[u] ? ex2(s[hh][u] - st.m) * kPScale : 0.f);
            st.l += (float)ph;
            const uint32_t ph2 = (uint32_t)__builtin_bit_cast(uint16_t, ph) * 0x00010001u;
            const half4_t bop = __builtin_bit_cast(half4_t, make_uint2(ph2 & ln.bmask0, ph2 & ln.bmask1));
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float4_t d = {st.acc[4 * i], st.acc[4 * i + 1], st.acc[4 * i + 2], st.acc[4 * i + 3]};
                d = __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(half4_t, av[u & 1][i]), bop, d, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) st.acc[4 * i + e] = d[e];
            }
        }
    }
}

// Launch modes.  kModeMulti: the launch holds several layers (the layer
// index comes from the workgroup index).  kModeByLength: one layer, one
// workgroup per (b, h), sequences taken longest first.  kModeOne: one layer,
// no ranking; a single-layer launch reads layer 0's operands at fixed
// argument offsets.  kModePair: like kModeOne, but a workgroup serves two
// consecutive query heads of one KV head (grouped-query attention): it reads
// each index row once and scores it against both heads' tables (see
// fold_pair).
constexpr int kModeOne = 0, kModeMulti = 1, kModeByLength = 2, kModePair = 3;

template <int S, int CG, typename CB, int kMode>
__global__ __launch_bounds__(kThreads) void decode_main(DecodeArgs a) {
    constexpr bool kMulti = kMode == kModeMulti;
    using Sh = Shape<S, CG, CB>;
    // query heads per workgroup; the second head's scores sit in the upper
    // half of every score-table row (one copy per row at S = 32)
    constexpr int NH = kMode == kModePair ? 2 : 1;
    static_assert(NH == 1 || (Sh::kMfma && Sh::KCOP == 1 && 2 * S == 64), "head pairs: the MFMA shape");
    constexpr int D = Sh::D, R = Sh::R, TPW = Sh::TPW;
    constexpr int NRD = Sh::NRD, CPR = Sh::CPR, G = Sh::G;
    constexpr int BSTEP = kWaves * TPW * kUnroll;   // tokens per batch of the workgroup
    static_assert(Sh::kLds <= kLdsLimit, "LDS budget");
    static_assert(D <= kThreads, "one thread per output channel");
    static_assert(2 * kMaxOrderedBatch <= kThreads, "the length ranking fits the reduction space");
    // The only LDS object: tables at byte 0 and 64K, then q, wave stats,
    // reduction partials and the arrival word.
    __shared__ __align__(16) unsigned char smem[Sh::kLds];
    float *qs = reinterpret_cast<float *>(smem + Sh::kBase);   // [NH][D]
    float *wstat = qs + NH * D;                 // [NH][kWaves][m, l]
    float *red = wstat + 2 * NH * kWaves;       // [G][D], or [NH][D]
    uint32_t *arrival = reinterpret_cast<uint32_t *>(red + kThreads);   // [NH]

    // The splits of one (layer, b, h) share an XCD (and its L2, which then
    // serves their table slices once); within the group, roles follow the
    // dispatch order (decode_role).  Layers are outermost.
    const unsigned p = blockIdx.x;
    const WgRole wr = decode_role(p, gridDim.x, (unsigned)a.n_split);
    const unsigned hgroups = (unsigned)a.H / NH;     // head groups per sequence
    const unsigned groups_per_layer = hgroups * a.B;
    const int layer = kMulti ? (int)(wr.group / groups_per_layer) : 0;
    const unsigned gq = kMulti ? wr.group % groups_per_layer : wr.group;
    const int split = wr.role;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int h = (int)(gq % hgroups) * NH, b = (int)(gq / hgroups);   // h: the first head
    if constexpr (kMode == kModeByLength) {
        // One workgroup per (b, h) over several rounds: the longest
        // sequences go first (in dispatch order), so the last round holds the
        // shortest ones.  Rank by (length descending, index ascending), a
        // permutation whatever the lengths are.
        h = (int)(p % a.H);
        int *lens = reinterpret_cast<int *>(red);
        int *order = lens + kMaxOrderedBatch;
        if (tid < a.B) lens[tid] = a.ctx_len[tid];
        __syncthreads();
        if (tid < a.B) {
            const int mine = lens[tid];
            int rank = 0;
            for (int i = 0; i < a.B; ++i) {
                const int li = lens[i];
                rank += (li > mine) | ((li == mine) & (i < tid));
            }
            order[rank] = tid;
        }
        __syncthreads();
        b = order[p / a.H];
    }
    const DecodeLayer &lp = a.layer[layer];
    const int tk = lane / R;
    Lanes<S, CG, CB> ln;
    ln.init(lane);
    const int r = ln.r;

    // Everything derived from the arguments, computed once up front so that
    // the argument and length loads form a single round trip.
    const int n_sink = a.n_sink, n_recent = a.n_recent, W = n_sink + n_recent;
    const int64_t t_max = a.t_max;
    const int Lraw = a.ctx_len[b];
    const int vqraw = a.vq_len ? a.vq_len[b] : -1;
    const size_t bh = (size_t)b * a.H + h;             // (first) query head: q, partials, out
    const int hk = h / a.q_per_kv;                      // KV head: caches, codebooks, windows
    const size_t bhk = (size_t)b * a.Hk + hk;
    const CB *kcb = static_cast<const CB *>(lp.kcb_t) + (size_t)hk * 256 * S * CG;
    const CB *vcb = static_cast<const CB *>(lp.vcb_t) + (size_t)hk * 256 * S * CG;
    const size_t wbase = (size_t)b * a.win_bstride + ((size_t)hk * W) * D;
    const uint16_t *kw = lp.kwin_t + wbase;
    const uint16_t *vw = lp.vwin_t + wbase;
    const uint8_t *kidx = lp.k_index + bhk * (size_t)t_max * S;
    const uint8_t *vidx = lp.v_index + bhk * (size_t)t_max * S;
    const uint32_t lane_off = (uint32_t)(tk * S + 8 * r);
    // the heads of a workgroup are consecutive, so are their workspace blocks
    // and output rows: head hh's block is blk + hh * kBlockBytes
    char *blk = a.blocks + ((size_t)layer * a.B * a.H + bh) * kBlockBytes;
    uint64_t *ticket = reinterpret_cast<uint64_t *>(blk);          // arrival word
    const uint64_t *parts = reinterpret_cast<const uint64_t *>(blk + kSlotBase);
    uint64_t *part = reinterpret_cast<uint64_t *>(blk + kSlotBase) + (size_t)split * (D + 2);
    float *outp = lp.out + bh * D;
    constexpr size_t kBlockWords = kBlockBytes / sizeof(uint64_t);
    const float scale = a.scale_log2;
    const int n_split = a.n_split;
    const int n_win = a.window_wg;
    const bool sep = n_win != 0;
    const int wi = split - (n_split - n_win);              // window workgroup index (sep)
    const bool vq_wg = !sep || wi < 0;                     // takes a VQ chunk

    // Loads that depend only on (b, h, t) go out first: q (raw bf16 bits,
    // converted later so that no wait is placed here) and the table slices.
    const uint32_t qraw = lp.q[bh * D + min(tid, NH * D - 1)];
    // bf16 codebooks: the q words this thread's part of the score table needs
    // (Stage::finish), so that each wave builds its part as soon as its own
    // loads are in, without a barrier for every wave's q
    uint32_t qk[NH][4];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
        uint4 w4 = make_uint4(0u, 0u, 0u, 0u);
        if constexpr (Sh::kF16V)
            w4 = *reinterpret_cast<const uint4 *>(lp.q + (bh + hh) * D + ((tid * Sh::EPU) % S) * CG);
        qk[hh][0] = w4.x; qk[hh][1] = w4.y; qk[hh][2] = w4.z; qk[hh][3] = w4.w;
    }
    // The block's epoch cannot change before this workgroup arrives, so it is
    // read now, overlapped with the prologue; it tags the partials.  Only the
    // epoch half of the arrival word is read (a 64-bit load whose low half is
    // dead would let the compiler reuse that register and wait for the load
    // before the index rows go out).
    uint32_t epoch_word = 0;                    // thread hh < NH: head hh's
    if (tid < NH && a.n_split > 1)
        epoch_word = __hip_atomic_load(reinterpret_cast<uint32_t *>(ticket + tid * kBlockWords) + 1,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    Stage<S, CG, CB> stg;
    {
        const int slice = vq_wg ? 256 * S * CG * (int)sizeof(CB) : 0;
        stg.load(__builtin_amdgcn_make_buffer_rsrc(const_cast<CB *>(kcb), (short)0, slice, kBufferWord3),
                 __builtin_amdgcn_make_buffer_rsrc(const_cast<CB *>(vcb), (short)0, slice, kBufferWord3));
    }

    // The first index batches are addressed from host-known values: a
    // sequence with any VQ token has L > n_sink + ..., so its VQ range starts
    // at n_sink.  Rows outside the range are masked later by the true range,
    // so these loads need not wait for the context length.
    // window rows of the first pass (wave w takes slots s0 + w + kWaves * (tk + pass * TPW))
    const int wr_idx = sep ? wi : split;                   // window range (sep: if >= 0)
    const int s0 = (sep && vq_wg) ? 0 : min(W, wr_idx * a.win_per);
    const int s1 = (sep && vq_wg) ? 0 : min(W, s0 + a.win_per);
    using Win = WindowPass<S, CG, CB>;
    // With at most 4 channels per sub-vector step a second pass's rows fit
    // the registers: pass p + 1 is in flight while pass p is folded.
    constexpr bool kWinDB = NH == 1 && CG <= 4;
    constexpr int WP = kWaves * TPW;             // window slots per pass
    int wslot = s0 + wave;
    Win win, win2;
    win.load(kw, vw, wslot + kWaves * tk, s1, ln);
    if constexpr (kWinDB) {
        if (wslot + WP < s1) win2.load(kw, vw, wslot + WP + kWaves * tk, s1, ln);
    }

    const int vq0 = n_sink + split * a.chunk;
    IndexRows ir0;                              // rows up to the end of the split's chunk
    ir0.init(kidx, vidx, vq_wg ? (int)min((int64_t)vq0 + a.chunk, t_max) : 0, lane_off, S);
    Batch r0, r1, r2;
    // The second batch waits: at start-up every workgroup's first loads queue
    // for HBM together, and the table slices, which gate the token loop, get
    // through sooner with fewer rows ahead of them.  With the rows of S >= 16
    // a wave issues it once its own part of the tables is built, otherwise
    // after the first barrier (measured: 32K at 0.25 bit 15.5 -> 15.3 us).
    constexpr bool kSecondAfterBuild = S >= 16;
    // The two waves of a SIMD issue their loads one after the other (waves
    // 0-3 first), and index rows, which miss to HBM, hold up the slice loads
    // queued behind them.  So in a launch of split heads (all workgroups
    // starting together) waves 0-3 issue their first batch too after their
    // part of the tables, behind waves 4-7's slices (measured: 32K, 0.5 bit,
    // 14.2-14.4 -> 13.9 us; 2-8 layers per launch -0.2 to -0.4 us; no gain
    // with head pairs).  Wave-uniform.
    const bool defer0 = kSecondAfterBuild && (kMode == kModeOne || kMode == kModeMulti) && n_split > 1 &&
                        wave < kWaves / 2;
    if (!defer0) load_batch<S, CG, CB>(ir0, vq0 + wave * TPW, r0);

    const Windows w = seq_windows(Lraw, vqraw, t_max, n_sink, n_recent);
    const int t0 = w.n_s + split * a.chunk;   // == vq0 whenever t0 < t1
    const int t1 = vq_wg ? min(t0 + a.chunk, w.n_s + w.n_v) : t0;
    int base = t0 + wave * TPW;
    IndexRows ir;                               // rows up to the end of the split's range
    ir.init(kidx, vidx, max(t1, 0), lane_off, S);

    const float qv = bf16f((uint16_t)qraw);
    if (tid < NH * D) qs[tid] = qv * scale;
    if (tid < NH) arrival[tid] = epoch_word;
    // q in LDS is read by the window passes and by fp32-codebook table builds;
    // a VQ workgroup with bf16 codebooks needs neither (the barrier is
    // workgroup-uniform)
    if (!Sh::kF16V || s0 < s1) __syncthreads();
    if constexpr (!kSecondAfterBuild) load_batch<S, CG, CB>(ir0, vq0 + wave * TPW + BSTEP, r1);

    // The window tokens need no table: where registers allow, fold them while
    // the table slices are still arriving, then build the tables.
    // (with two heads the window rows wait for the build: their registers
    // and the staged slices would not fit together)
    constexpr bool kWindowFirst = NH == 1 && Sh::NACC <= 32;
    Online<Sh::NACC> sts[NH];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) sts[hh].init();
    Online<Sh::NACC> &st = sts[0];
    // Build the tables.  A value codebook entry outside fp16's range is
    // flagged in the status word.  The VQ workgroups of a head stage the same
    // slice, so they share that check: the one of VQ role `split` among
    // n_vq_wg checks the staged units u with u = split (mod nq),
    // nq = min(n_vq_wg, 8), as they are converted.
    const int n_vq_wg = n_split - n_win;
    uint32_t check_units = 0;
    {
        const int nq = n_vq_wg < 8 ? n_vq_wg : 8;
        for (int u = split % nq; u < Sh::UPT; u += nq) check_units |= 1u << u;
    }
    auto build_tables = [&]() {
        const bool bad = stg.template finish<NH>(qs, qk, scale, smem, check_units);
        if constexpr (Sh::kF16V) {
            if (__ballot(bad) != 0 && lane == 0)
                __hip_atomic_fetch_or(a.status, kStatusValueRange, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    };
    if constexpr (!kWindowFirst) {
        if (vq_wg) {
            build_tables();
            if constexpr (kSecondAfterBuild) {
                if (defer0) load_batch<S, CG, CB>(ir0, vq0 + wave * TPW, r0);
                load_batch<S, CG, CB>(ir0, vq0 + wave * TPW + BSTEP, r1);
            }
        }
        __syncthreads();
    }
    if constexpr (NH == 2) {
        while (wslot < s1) {                     // wave-uniform
            win.fold_pair(qs, sts, r, w, n_sink, n_recent);
            wslot += WP;
            if (wslot < s1) win.load(kw, vw, wslot + kWaves * tk, s1, ln);
        }
    } else if constexpr (kWinDB) {
        while (wslot < s1) {                     // wave-uniform
            win.fold(qs, st, r, w, n_sink, n_recent);
            wslot += WP;
            if (wslot + WP < s1) win.load(kw, vw, wslot + WP + kWaves * tk, s1, ln);
            if (wslot >= s1) break;
            win2.fold(qs, st, r, w, n_sink, n_recent);
            wslot += WP;
            if (wslot + WP < s1) win2.load(kw, vw, wslot + WP + kWaves * tk, s1, ln);
        }
    } else {
        while (wslot < s1) {                     // wave-uniform
            win.fold(qs, st, r, w, n_sink, n_recent);
            wslot += WP;
            if (wslot < s1) win.load(kw, vw, wslot + kWaves * tk, s1, ln);
        }
    }
    if constexpr (kWindowFirst) {
        if (vq_wg) {
            build_tables();
            if constexpr (kSecondAfterBuild) {
                if (defer0) load_batch<S, CG, CB>(ir0, vq0 + wave * TPW, r0);
                load_batch<S, CG, CB>(ir0, vq0 + wave * TPW + BSTEP, r1);
            }
        }
        __syncthreads();
    }
    // Waves w and w + 4 share a SIMD; the older one would win every issue slot
    // and finish long before its partner.  Their priorities alternate from
    // batch to batch instead, so both reach the reduction together.
    int turn = __builtin_amdgcn_readfirstlane(wave >> 2);
    auto take_turn = [&]() {
        if (turn & 1)
            __builtin_amdgcn_s_setprio(1);
        else
            __builtin_amdgcn_s_setprio(0);
        ++turn;
    };
    auto fold_next = [&](const Batch &bt) {
        if constexpr (NH == 2)
            fold_pair<S, CG, CB>(bt, base, t1, smem, ln, sts);
        else
            fold_batch<S, CG, CB>(bt, base, t1, smem, ln, st);
    };
    // three-deep ring, unrolled so that every batch lives in named registers
    while (true) {                               // wave-uniform
        if (base >= t1) break;
        load_batch<S, CG, CB>(ir, base + 2 * BSTEP, r2);
        take_turn();
        fold_next(r0);
        base += BSTEP;
        if (base >= t1) break;
        load_batch<S, CG, CB>(ir, base + 2 * BSTEP, r0);
        take_turn();
        fold_next(r1);
        base += BSTEP;
        if (base >= t1) break;
        load_batch<S, CG, CB>(ir, base + 2 * BSTEP, r1);
        take_turn();
        fold_next(r2);
        base += BSTEP;
    }
    __builtin_amdgcn_s_setprio(0);

    // Lane accumulators to the freed table space: row (wave, tk), natural
    // channel order.  Then wave (m, l).
    // per head: the wave's l (every token was counted R times), the block's
    // epoch (0 .. kEpochWrap - 1) and the call's tag (never 0: zero-filled
    // slots)
    float lwh[NH];
    uint32_t epochh[NH], tagh[NH];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
        lwh[hh] = wave_sum(sts[hh].l) * (1.f / R);
        epochh[hh] = arrival[hh];
        tagh[hh] = epochh[hh] + 1u;
    }
    const int n = n_split;
    // MFMA layout: token slots tk and tk + TPW/2 (lanes 32 apart) have the
    // same rotation, so their accumulators hold the same channels.  One lane
    // swap and an add per pair of accumulators fold them while other waves
    // are still in their loops: lanes 0-31 keep the sums of blocks 0-3 (the
    // first operand), lanes 32-63 those of blocks 4-7.
    float fold[NH][Sh::kMfma ? 16 : 1];
    if constexpr (Sh::kMfma) {
        static_assert(D == 128 && R == 4 && TPW == 16, "one MFMA shape");
#pragma unroll
        for (int hh = 0; hh < NH; ++hh)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(sts[hh].acc[4 * i + e]),
                                                                     __float_as_uint(sts[hh].acc[4 * (i + 4) + e]),
                                                                     false, false);
                    fold[hh][4 * i + e] = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
                }
    }
    // Plain value sums, folded slots: one lane swap and an add per pair of
    // accumulators a, a + NACC/2 leave lanes 0-31 with sub-vector steps 0-3
    // (the first half of the array) and lanes 32-63 with steps 4-7.
    constexpr bool kFoldPlain = Sh::kFold && !Sh::kMfma;
    float foldp[kFoldPlain ? Sh::NACC / 2 : 1];
    if constexpr (kFoldPlain) {
        static_assert(NH == 1 && Sh::NACC == 8 * NRD * CPR, "one head, 8 steps of NRD reads");
#pragma unroll
        for (int k = 0; k < Sh::NACC / 2; ++k) {
            const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(st.acc[k]),
                                                             __float_as_uint(st.acc[k + Sh::NACC / 2]), false, false);
            foldp[k] = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
        }
    }
    __syncthreads();                             // every wave is done with the tables
    // Who merges.  With window workgroups (the grid fits the chip) it is the
    // last of them: it has the highest index of its (b, h), so its peers were
    // dispatched before it, and it is done early, so it simply waits for
    // their partials.  Otherwise the last workgroup to take an arrival ticket
    // merges; the ticket travels while the partial is reduced.
    uint64_t ticket_word = 0;
    if (NH == 1 && tid == 0 && n > 1 && !sep)
        ticket_word = __hip_atomic_fetch_add(ticket, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    float *dump = reinterpret_cast<float *>(smem);
    constexpr int RPW = Sh::NR / kWaves;        // dump rows per wave
    const int drow = wave * RPW + tk % RPW;
    if constexpr (Sh::kQuadRed) {
        // 16-byte (or 8-byte) pieces at padded rows.  MFMA layout: the lane's
        // accumulators 4i .. 4i + 3 (rows e of its block) hold channels
        // 32e + q, q = 4 ((i + rot) mod 8) + r, stored at position 4q + e;
        // otherwise positions are channels.
        unsigned char *rowp = smem + (size_t)drow * Sh::RS;
        if constexpr (Sh::kMfma) {
            // head hh's rows follow the first head's NR rows
            const int hb = lane >> 5;            // folded blocks 4 hb .. 4 hb + 3
#pragma unroll
            for (int hh = 0; hh < NH; ++hh)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *reinterpret_cast<float4 *>(rowp + (size_t)hh * Sh::NR * Sh::RS +
                                                16 * (4 * ((i + 4 * hb + ln.rot) & 7) + r)) =
                        make_float4(fold[hh][4 * i], fold[hh][4 * i + 1], fold[hh][4 * i + 2], fold[hh][4 * i + 3]);
        } else {
            // folded: this lane's steps i0 .. i0 + 3
            constexpr int NI = kFoldPlain ? 4 : 8;
            const int i0 = kFoldPlain ? (lane >> 5) * 4 : 0;
            const float *accs = kFoldPlain ? foldp : st.acc;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
#pragma unroll
                for (int hh = 0; hh < NRD; ++hh) {
                    const float *acc = accs + (i * NRD + hh) * CPR;
                    float *dst = reinterpret_cast<float *>(rowp) + ln.channel(i0 + i, hh);
                    if constexpr (CPR == 4)
                        *reinterpret_cast<float4 *>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
                    else
                        *reinterpret_cast<float2 *>(dst) = make_float2(acc[0], acc[1]);
                }
            }
        }
    } else {
        static_assert(!Sh::kMfma, "MFMA value sums come with head_dim 128");
        float *mine = dump + (size_t)drow * D;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
            for (int hh = 0; hh < NRD; ++hh) {
                const float *acc = st.acc + (i * NRD + hh) * CPR;
                float *dst = mine + ln.channel(i, hh);
                if constexpr (CPR == 4)
                    *reinterpret_cast<float4 *>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
                else
                    *reinterpret_cast<float2 *>(dst) = make_float2(acc[0], acc[1]);
            }
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
            wstat[2 * (hh * kWaves + wave)] = sts[hh].m;
            wstat[2 * (hh * kWaves + wave) + 1] = lwh[hh];
        }
    }
    __syncthreads();

    // Workgroup partial: scale every wave to the common max (empty waves have
    // l == 0 and zero accumulators) and sum the dumped rows.
    float ewh[NH][kWaves], Mh[NH], lth[NH];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
        float mw[kWaves], lv[kWaves];
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            mw[v] = wstat[2 * (hh * kWaves + v)];
            lv[v] = wstat[2 * (hh * kWaves + v) + 1];
        }
        float Mx = -INFINITY;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) Mx = lv[v] > 0.f ? fmaxf(Mx, mw[v]) : Mx;
        float lx = 0.f;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            ewh[hh][v] = lv[v] > 0.f ? ex2(mw[v] - Mx) : 0.f;
            lx += lv[v] * ewh[hh][v];
        }
        Mh[hh] = Mx;
        lth[hh] = lx;
    }
    const float *ew = ewh[0];
    if constexpr (Sh::kQuadRed) {
        // thread (q, s): positions 4q .. 4q + 3 of rows s, s + SS, ...; the
        // SS subsets of a quad are consecutive lanes, summed with DPP (and one
        // lane exchange when SS = 32)
        constexpr int QD = D / 4, SS = kThreads / QD, RPT = Sh::NR / SS;
        static_assert(SS == 16 || SS == 32, "subsets fill DPP rows");
        const int sb = tid % SS, q = tid / SS;
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
        float4 a4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int row = sb + SS * i;
            // the row's wave, among the few a row of this i can belong to
            float sc = ewh[hh][(SS * i) / RPW];
#pragma unroll
            for (int w = (SS * i) / RPW + 1; w <= (SS * i + SS - 1) / RPW; ++w)
                if (row >= w * RPW) sc = ewh[hh][w];
            const float4 v = *reinterpret_cast<const float4 *>(smem + (size_t)(hh * Sh::NR + row) * Sh::RS + 16 * q);
            a4.x += sc * v.x;
            a4.y += sc * v.y;
            a4.z += sc * v.z;
            a4.w += sc * v.w;
        }
        a4.x = row_sum(a4.x);
        a4.y = row_sum(a4.y);
        a4.z = row_sum(a4.z);
        a4.w = row_sum(a4.w);
        if constexpr (SS == 32) {
            float p0, p1;
            pair16(a4.x, p0, p1); a4.x = p0 + p1;
            pair16(a4.y, p0, p1); a4.y = p0 + p1;
            pair16(a4.z, p0, p1); a4.z = p0 + p1;
            pair16(a4.w, p0, p1); a4.w = p0 + p1;
        }
        if (sb == 0) {
            const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) red[hh * D + (Sh::kMfma ? 32 * e + q : 4 * q + e)] = av[e];
        }
      }
    } else {
        const int ch = tid % D, g = tid / D;
        float acc = 0.f;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            float sv = 0.f;
#pragma unroll
            for (int qq = 0; qq < TPW / G; ++qq) sv += dump[(size_t)(v * TPW + g + qq * G) * D + ch];
            acc += sv * ew[v];
        }
        red[g * D + ch] = acc;
    }
    __syncthreads();
    // Thread tid < NH * D owns channel tid % D of head hme = tid / D (the
    // heads' output rows and workspace blocks are consecutive).
    const int hme = tid / D < NH ? tid / D : NH - 1;
    const float M = Mh[hme], lt = lth[hme];
    const uint32_t tag = tagh[hme];
    float o = 0.f;
    if (tid < NH * D) {
        if constexpr (Sh::kQuadRed) {
            o = red[tid];
        } else {
#pragma unroll
            for (int g = 0; g < G; ++g) o += red[g * D + tid];
        }
    }
    // One workgroup per (b, h): nothing to merge, and the workspace is not
    // touched.
    if (n == 1) {
        if (tid < NH * D) outp[tid] = lt > 0.f ? o / lt : 0.f;
        return;
    }
    uint64_t *const part_me = part + hme * kBlockWords;
    // Every workgroup publishes at once (before it knows whether it is last,
    // so the others' pairs are already on their way when the last one looks).
    if (sep) {
        if (split != n - 1) {                    // token splits publish and leave
            if (tid < NH * D) publish(&part_me[2 + tid % D], o, tag);
            if (tid < NH * D && tid % D == 0) {
                publish(&part_me[0], M, tag);
                publish(&part_me[1], lt, tag);
            }
            return;
        }
    } else if constexpr (NH == 2) {
        return;                                  // (never launched: head pairs use window workgroups)
    } else {
        if (tid < D) publish(&part[2 + tid], o, tag);
        if (tid == 0) {
            publish(&part[0], M, tag);
            publish(&part[1], lt, tag);
            *arrival = (uint32_t)ticket_word;            // arrivals before this one
        }
        __syncthreads();
        if ((int)*arrival != n - 1) return;
    }

    // The merger: every other workgroup of (b, h) has started (and will
    // publish); poll their pairs (slot `split` is this workgroup's own).
    // Threads below NH * D own a channel (of head hme: with two heads, waves
    // 0-1 merge the first, waves 2-3 the second); at least 32 take part (the
    // per-slot m and l pairs are read by lanes 0..31).
    constexpr int kMergeThreads = NH * D > 32 ? NH * D : 32;
    if (tid >= kMergeThreads) return;
    const int ch = tid < NH * D ? tid % D : 0;
    const uint64_t *const parts_me = parts + hme * kBlockWords;
    // slots in ascending order, this workgroup's own (slot `split`) from its
    // registers: the same sum whichever workgroup merges
    float Mg = -INFINITY;
    float num = 0.f, den = 0.f;
    bool failed = false;
    // A poll reads this channel of every slot of a chunk, and one (m or l)
    // pair per lane: lane i of a 32-lane half reads m of slot i (i < 16) or l
    // of slot i - 16.  One poll is in flight at a time: a second one, issued
    // half a round trip later, sees the last partial sooner, but the wave
    // cannot end before its loads land, so the call would not end sooner.
    static_assert(kMergeChunk == 16, "a chunk's m and l pairs fill one 32-lane half");
    struct Poll {
        uint64_t po[kMergeChunk];
        uint64_t ml;
    };
    const int hl = tid & 31;
    for (int c0 = 0; c0 < n; c0 += kMergeChunk) {
        auto issue = [&](Poll &pp) {
#pragma unroll
            for (int i = 0; i < kMergeChunk; ++i) {
                const size_t sl = (size_t)min(c0 + i, n - 1) * (D + 2);
                pp.po[i] = __hip_atomic_load(&parts_me[sl + 2 + ch], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            const size_t sl = (size_t)min(c0 + (hl & 15), n - 1) * (D + 2);
            pp.ml = __hip_atomic_load(&parts_me[sl + (hl >> 4)], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        };
        // branch-free: a slot counts if it exists and is not this workgroup's
        auto current = [&](const Poll &pp) {
            uint32_t ok = 1u;
#pragma unroll
            for (int i = 0; i < kMergeChunk; ++i) {
                const uint32_t want = (uint32_t)(c0 + i < n) & (uint32_t)(c0 + i != split);
                ok &= (uint32_t)((uint32_t)(pp.po[i] >> 32) == tag) | (want ^ 1u);
            }
            const int si = c0 + (hl & 15);
            const uint32_t want = (uint32_t)(si < n) & (uint32_t)(si != split);
            ok &= (uint32_t)((uint32_t)(pp.ml >> 32) == tag) | (want ^ 1u);
            return __all(ok != 0u);
        };
        // merge a chunk from the poll that saw every pair current.  The slot
        // weights are computed one slot per lane: lane i of a 32-lane half
        // holds m of slot c0 + i (i < 16), lane i + 16 its l; after the
        // exchange every 16-lane row holds all 16 slots, so row reductions
        // (however many rows are active) give the chunk's max and weight sum.
        auto merge = [&](const Poll &pp) {
            const float v = __uint_as_float((uint32_t)pp.ml);
            const float vo = __shfl_xor(v, 16);
            const int si = c0 + (hl & 15);
            const bool own = si == split;
            const float ms = own ? M : (hl < 16 ? v : vo), ls = own ? lt : (hl < 16 ? vo : v);
            const bool use = (si < n) & (ls > 0.f);
            const float mi = use ? ms : -INFINITY;
            const float mc = fmaxf(Mg, row_max(mi));
            if (mc > Mg) {                           // Mg = -inf gives 0 * 0
                const float sc = Mg == -INFINITY ? 0.f : ex2(Mg - mc);
                num *= sc;
                den *= sc;
                Mg = mc;
            }
            const float e = use ? ex2(mi - Mg) : 0.f;
            den += row_sum(use ? ls * e : 0.f);
#pragma unroll
            for (int i = 0; i < kMergeChunk; ++i)
                num += (c0 + i == split ? o : __uint_as_float((uint32_t)pp.po[i])) * lane_f(e, i);
        };
        Poll pa;
        int poll = 0;
        while (true) {
            issue(pa);
            if (current(pa)) {
                merge(pa);
                break;
            }
            if (++poll >= a.max_polls) {
                failed = true;
                break;
            }
        }
    }
    // (a timed-out merge writes quiet-NaN bits: an integer select, so that the
    // no-NaN arithmetic this file is built with cannot fold it away) and is
    // flagged in the status word
    if (tid < NH * D)
        reinterpret_cast<uint32_t *>(outp)[tid] =
            failed ? 0x7fc00000u : __float_as_uint(den > 0.f ? num / den : 0.f);
    if (tid < NH * D && ch == 0) {
        if (failed) __hip_atomic_fetch_or(a.status, kStatusMergeTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t epoch = epochh[hme];
        const uint32_t next = epoch + 1u == kEpochWrap ? 0u : epoch + 1u;
        __hip_atomic_store(ticket + hme * kBlockWords, (uint64_t)next << 32, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int S, int CG, typename CB>
constexpr bool fits() {
    if constexpr (S * CG * (std::is_same<CB, uint16_t>::value ? 2 : 4) > 256) return false;
    else return Shape<S, CG, CB>::kLds <= kLdsLimit;
}

template <int S, int CG>
hipError_t launch_sc(const DecodeArgs &a, hipStream_t st) {
    const dim3 grid((unsigned)a.n_split * (a.H / a.heads_per_wg) * a.B * a.n_layers);
    const int mode = a.heads_per_wg == 2 ? kModePair
                     : a.n_layers > 1    ? kModeMulti
                     : a.by_length       ? kModeByLength
                                         : kModeOne;
    if (a.cb_bf16) {
        if constexpr (fits<S, CG, uint16_t>()) {
            if (mode == kModePair) {
                if constexpr (Shape<S, CG, uint16_t>::kMfma && Shape<S, CG, uint16_t>::KCOP == 1)
                    hipLaunchKernelGGL((decode_main<S, CG, uint16_t, kModePair>), grid, dim3(kThreads), 0, st, a);
                else
                    return hipErrorInvalidValue;
            } else if (mode == kModeMulti)
                hipLaunchKernelGGL((decode_main<S, CG, uint16_t, kModeMulti>), grid, dim3(kThreads), 0, st, a);
            else if (mode == kModeByLength)
                hipLaunchKernelGGL((decode_main<S, CG, uint16_t, kModeByLength>), grid, dim3(kThreads), 0, st, a);
            else
                hipLaunchKernelGGL((decode_main<S, CG, uint16_t, kModeOne>), grid, dim3(kThreads), 0, st, a);
        } else {
            return hipErrorInvalidValue;
        }
    } else {
        if constexpr (fits<S, CG, float>()) {
            if (mode == kModePair)
                return hipErrorInvalidValue;
            else if (mode == kModeMulti)
                hipLaunchKernelGGL((decode_main<S, CG, float, kModeMulti>), grid, dim3(kThreads), 0, st, a);
            else if (mode == kModeByLength)
                hipLaunchKernelGGL((decode_main<S, CG, float, kModeByLength>), grid, dim3(kThreads), 0, st, a);
            else
                hipLaunchKernelGGL((decode_main<S, CG, float, kModeOne>), grid, dim3(kThreads), 0, st, a);
        } else {
            return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

constexpr int kMaxDevices = 64;

}  // namespace

hipError_t scratch_address(hipStream_t stream, void **addr) {
    static std::mutex mu;
    static void *cached[kMaxDevices] = {};
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    int dev = cur;
    if (stream) {
        e = hipStreamGetDevice(stream, &dev);
        if (e != hipSuccess) return e;
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!cached[dev]) {
        // the address is per device: look it up with that device current
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        cached[dev] = ptr;
    }
    *addr = cached[dev];
    return hipSuccess;
}

bool decode_supported(int d, int S, int cg, int cb_bf16) {
#define LVQ_FIT(S_, CG_) \
    if (S == S_ && cg == CG_) return cb_bf16 ? fits<S_, CG_, uint16_t>() : fits<S_, CG_, float>();
    if (S * cg != d) return false;
    LVQ_FIT(8, 2)
    LVQ_FIT(8, 4)
    LVQ_FIT(8, 8)
    LVQ_FIT(16, 2)
    LVQ_FIT(16, 4)
    LVQ_FIT(16, 8)
    LVQ_FIT(32, 2)
    LVQ_FIT(32, 4)
    LVQ_FIT(64, 2)
#undef LVQ_FIT
    return false;
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t st) {
#define LVQ_CASE(S_, CG_) \
    if (a.S == S_ && a.cg == CG_) return launch_sc<S_, CG_>(a, st);
    LVQ_CASE(8, 2)
    LVQ_CASE(8, 4)
    LVQ_CASE(8, 8)
    LVQ_CASE(16, 2)
    LVQ_CASE(16, 4)
    LVQ_CASE(16, 8)
    LVQ_CASE(32, 2)
    LVQ_CASE(32, 4)
    LVQ_CASE(64, 2)
#undef LVQ_CASE
    return hipErrorInvalidValue;
}

}  // namespace lvq
