// LoopVQ encoder, gfx950: nearest codeword of every loop-stacked sub-vector.
//
// LoopVQ project page (mscheong01.github.io/loopvq), "Component 1 --
// Loop-axis vector quantization" and "Serving in SGLang -- Encode in pages";
// news article (notatechguy.com), "How LoopVQ works".  A sub-vector of
// (token n, head h, sub-vector j) has G = Tc * cg entries
// x_i = x[n][h][t][j*cg + c], i = t*cg + c; its code is
//     argmin_k D_k,  D_k = sum_i (x_i - c_{k,i})^2
// in IEEE fp32 (separate subtract, square, add; ascending i), lowest k on ties.
//
// Layout of the work.  A workgroup owns 4 sub-vectors j (one wave each) of one
// head and a chunk of tokens.  It first stages the 4 codebooks (all Tc
// slices, all 256 codes; the storage is code-major, so each (slice, code) row
// piece is one contiguous read) in LDS, with their squared norms, and builds
// the MFMA operands from them; that LDS then holds the chunk's codes on their
// way out.
//
// Screen (MFMA).  The screen value S_k = |c_k|^2 - 2 x.c_k differs from D_k by
// |x|^2, the same for every k.  MFMAs multiply 32 codes (rows) by 32 tokens
// (columns) over the K axis
//     code row  = [-2 c_k (split into P bf16 parts), 0...]
//     token col = [ x (repeated P times),           0...]
// (for fp32 codebooks c = c0 + c1 + c2 in bf16 parts, P = 3; bf16 codebooks
// P = 1), starting from the accumulator C = fl32(|c_k|^2): one
// v_mfma_f32_32x32x16_bf16 per 16 entries of K (one at the 0.5-bit shape,
// P G = 16).  Products of bf16 values are exact in fp32, so the only screen
// errors are the accumulation roundings.  Each wave keeps its codebook in
// registers as MFMA A operands and streams 32-token tiles through it; a token
// sits on two lanes (col, col + 32), each with 128 of its 256 codes.
// Each lane finds the two smallest screen values of its 128 codes from two
// partitions of them (16 groups of 8 codes, half an MFMA block each, and 8
// chains of 16; a group and a chain share one code): the minimum of every
// group and every chain (min3, two new values an instruction), then the two
// smallest group minima and the two smallest chain minima.  The smallest
// value is the smallest of either list, the second smallest the smaller of
// the two lists' second entries.  The low 4 bits of the group minima and the
// low 3 bits of the chain minima are replaced by their group or chain, so the
// smallest value names its code (the lane supplies the rest of the index).
//
// Exactness.  With R = |x| + max_k |c_k|, the (at most 4) bits written into a
// value move it by at most 2^-19 R^2; the fp32 error of D_k is at most
// (G+2) 2^-24 R^2 and that of the screen (C plus P*G exact products) at most
// F (P*G+3) 2^-24 R^2 for an accumulation F times worse than a sequential
// fp32 sum (P*G+1 terms; the bound keeps two terms of slack; any fp32
// summation order, rounded to nearest or truncated, has F <= 2).  If the two
// smallest (marked) screen values are more than eps apart, eps exceeds twice
// the sum of these, so the screen winner is the exact winner.  eps is
// 2^-16 R^2 where that still holds for F up to 3 or more (4.1 at G = 16 and
// 7.8 at G = 8 with P = 1, 3.2 at G = 8 with P = 3), else 2^-15 R^2 (5.4 at
// G = 32 with P = 1, 4.0 at G = 16 with P = 3).  (Where the group and the
// chain of a lane's smallest value would name different codes, two of its
// values are within a few marks of each other, so the test fails.)
// Otherwise the wave re-scores all 256 codes of that sub-vector exactly as
// defined above (64 lanes x 4 codes, strict < per lane in ascending k, then a
// lowest-index argmin across lanes), which reproduces the definition bit for
// bit; with bf16 codebooks the codewords come from the wave's MFMA operands
// (-2c, exact), with fp32 codebooks from the codebooks staged in LDS again.
#include "kernels.h"

#include <math.h>

#pragma clang fp contract(off)

namespace lvq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;     // 4 waves, one sub-vector index j each
constexpr int kJW = 4;            // sub-vectors per workgroup
constexpr int kTokChunk = 2048;   // tokens per workgroup
// eps / R^2 for G-entry sub-vectors and P-part codewords: eps = 256 units of
// 2^-24 R^2 when the marks (2 x 32), the exact distances (2 (G + 2)) and a
// screen with F = 3 (2 x 3 (P G + 3)) fit in it, else 512 units
template <int G, int P>
constexpr float eps_scale() {
    return 2 * 32 + 2 * (G + 2) + 2 * 3 * (P * G + 3) <= 256 ? 1.52587890625e-05f   // 2^-16
                                                              : 3.0517578125e-05f;  // 2^-15
}
constexpr uint16_t kRescore = 0x100;

__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// round-to-nearest-even fp32 -> bf16 bits (finite inputs)
__device__ __forceinline__ uint16_t bf16_rne(float v) {
    uint32_t u = __float_as_uint(v);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// part p (0, 1, 2) of the 3-way bf16 split of v: v ~= part0 + part1 + part2
__device__ __forceinline__ float split_part(float v, int p) {
    const float h0 = bf16f(bf16_rne(v));
    if (p == 0) return h0;
    const float r1 = v - h0;
    const float h1 = bf16f(bf16_rne(r1));
    if (p == 1) return h1;
    return bf16f(bf16_rne(r1 - h1));
}

template <typename CB>
__device__ __forceinline__ float to_f(CB v);
template <>
__device__ __forceinline__ float to_f<float>(float v) { return v; }
template <>
__device__ __forceinline__ float to_f<uint16_t>(uint16_t v) { return bf16f(v); }

// Cross-lane exchanges without LDS.  After pair16(x, a, b), {a, b} of every
// lane hold x of that lane and of lane ^ 16 (pair32: lane ^ 32), so any
// symmetric combination of a and b is the pairwise result in both lanes.
__device__ __forceinline__ void pair16(float x, float &a, float &b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void pair32(float x, float &a, float &b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}

// minimum over the 64 lanes, in every lane: DPP xor 1, xor 2, half-row and
// row mirrors within 16 lanes, then the two lane swaps
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false));
    auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = min(r[0], r[1]);
    r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return min(r[0], r[1]);
}

template <int G, int CG, int P, typename CB>
struct EncShape {
    static constexpr int T = G / CG;                       // loop steps
    static constexpr int KX = P * G;                       // K entries that carry x
    static constexpr int KC = 16;                          // K entries per 32x32x16 MFMA
    static constexpr int NCH = (KX + KC - 1) / KC;         // MFMAs per 32 codes x 32 tokens
    static constexpr int KL = KC / 2;                      // K entries per lane per MFMA
    static constexpr int LE = CG < KL ? CG : KL;           // x elements per load
    static constexpr int NLD = KL / LE;                    // loads per lane per MFMA
    static constexpr int EB = (int)sizeof(CB);
    static constexpr int ROWB = kJW * CG * EB;             // bytes of one (slice, code) row piece
    static constexpr int EC = 16 / EB;                     // elements per 16-byte chunk
    static constexpr int CHUNKS = T * 256 * ROWB / 16;     // staging chunks
    static_assert(ROWB % 16 == 0 && CHUNKS % kThreads == 0, "staging tiles");
    static_assert(G % 8 == 0 && (P * G) % 8 == 0, "operand blocks of 8");
};

// One 32-token tile of x as MFMA B-operand words: lane (col, hf) holds, for
// each K chunk ch, the KL/2 words (KL bf16) of entries kk = ch*KC + hf*KL ..
// + KL - 1 of token n0 + col (zero where kk is not an x entry or the token is
// past the end).
template <int NCH, int KL>
struct XTile {
    uint32_t w[NCH][KL / 2];
};

constexpr uint32_t kOob = 0xffffff00u;            // offset past any buffer: loads return 0
constexpr int kBufferWord3 = 0x00020000;          // raw buffer resource, gfx9 family

// NLD loads of LE x elements per lane and MFMA (offsets from the tile base)
template <int NCH, int KL, int LE>
__device__ __forceinline__ void load_tile(XTile<NCH, KL> &t, __amdgpu_buffer_rsrc_t rs,
                                          const uint32_t (&off)[NCH][KL / LE], bool valid) {
    constexpr int NLD = KL / LE;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
        for (int s = 0; s < NLD; ++s) {
            const uint32_t o = valid ? off[ch][s] : kOob;
            if constexpr (LE == 8) {
                const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, 0));
                t.w[ch][0] = v.x; t.w[ch][1] = v.y; t.w[ch][2] = v.z; t.w[ch][3] = v.w;
            } else if constexpr (LE == 4) {
                const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, o, 0, 0));
                t.w[ch][2 * s] = v.x; t.w[ch][2 * s + 1] = v.y;
            } else {
                t.w[ch][s] = __builtin_amdgcn_raw_buffer_load_b32(rs, o, 0, 0);
            }
        }
    }
}

typedef float floatx16 __attribute__((ext_vector_type(16)));

// acc = A * B + acc for one K chunk of 16: lane (col, hf) supplies A[col][8 hf
// .. 8 hf + 7] and B[8 hf .. 8 hf + 7][col]; it receives D[8 (v / 4) + 4 hf +
// v % 4][col] in acc[v]
__device__ __forceinline__ floatx16 mfma_chunk(const uint32_t *aw, const uint32_t *bw, floatx16 acc) {
    const bf16x8 A = __builtin_bit_cast(bf16x8, make_uint4(aw[0], aw[1], aw[2], aw[3]));
    const bf16x8 B = __builtin_bit_cast(bf16x8, make_uint4(bw[0], bw[1], bw[2], bw[3]));
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, acc, 0, 0, 0);
}

// Parts the codebooks are staged in: with bf16 codebooks of 32 entries (64
// KiB for the 4 sub-vectors) two parts of 2, where a part's row pieces are
// whole 16-byte reads, so that 3 workgroups fit a compute unit's LDS.
template <int G, int CG, int P, typename CB>
constexpr int staging_parts() {
    return P == 1 && G > 16 && (kJW / 2 * CG * (int)sizeof(CB)) % 16 == 0 ? 2 : 1;
}

// kScreen: also store every unmarked screen value to a.screen (the
// diagnostic entry point that measures the screen's error; the values, the
// operands and the instructions that form them are those of the plain
// instance)
template <int G, int CG, int P, typename CB, bool kScreen>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(
    kScreen ? 1 : G * P <= 16 ? 4 : staging_parts<G, CG, P, CB>() == 2 ? 3 : 1))) void
encode_kernel(EncodeArgs a) {
    using Sh = EncShape<G, CG, P, CB>;
    constexpr int NCH = Sh::NCH;
    // The staged codebooks [jl][k][i] are read only until the MFMA operands
    // are built; then the same LDS holds, per wave, the code of each chunk
    // row or kRescore (re-score it exactly).  Sharing the space lets more
    // workgroups fit a compute unit.  Each staged part is read by its waves
    // before the next replaces it.
    constexpr int kParts = staging_parts<G, CG, P, CB>();
    constexpr int kJP = kJW / kParts;                             // sub-vectors per part
    constexpr int kCbBytes = kJP * 256 * G * (int)sizeof(CB);
    constexpr int kCodeBytes = kJW * kTokChunk * 2;
    constexpr int kMarkWords = kTokChunk / 32;                    // one word per 32-token tile
    constexpr int kMarkBytes = kJW * kMarkWords * 4;
    __shared__ __align__(16) unsigned char
        stage[kCbBytes > kCodeBytes + kMarkBytes ? kCbBytes : kCodeBytes + kMarkBytes];
    __shared__ float nrm[kJW * 256];
    CB *cbs = reinterpret_cast<CB *>(stage);
    uint16_t(*row_code)[kTokChunk] = reinterpret_cast<uint16_t(*)[kTokChunk]>(stage);
    // (the wave index is uniform; saying so keeps the buffer resources built
    // from it in scalar registers)
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // grid z = tensor * H + head (a launch may encode two tensors, e.g. K and V)
    // One linear grid over (tensor * H + head, token chunk, group of kJW
    // sub-vectors), the group fastest.  Workgroups are dealt to the 8 XCDs in
    // turn (dispatch d to XCD d % 8), so XCD k takes a contiguous run of the
    // linear index: the workgroups of a chunk that cover the groups of one
    // input row (32 bytes of it each) and fill its index rows (4 bytes each)
    // start together on one XCD and share its L2.
    const int ny = (a.S + kJW - 1) / kJW;
    const int nchunk = (int)((a.n_tokens + kTokChunk - 1) / kTokChunk);
    const int n_wg = nchunk * ny * a.H * a.n_tensors;
    const int dsp = (int)blockIdx.x, xcd = dsp % 8, per = n_wg / 8, rem = n_wg % 8;
    const int lin = xcd * per + min(xcd, rem) + dsp / 8;
    const int yg = lin % ny, chunk = (lin / ny) % nchunk, zz = lin / (ny * nchunk);
    const int tz = zz / a.H;
    const int h = zz - tz * a.H;
    const uint16_t *xin = tz ? a.x_b : a.x;
    const void *cbin = tz ? a.cb_b : a.cb;
    uint8_t *idxout = tz ? a.index_b : a.index;
    const int j0 = yg * kJW, j = j0 + wave;
    const int64_t tok0 = (int64_t)chunk * kTokChunk;
    const int64_t tok_end = min(tok0 + kTokChunk, a.n_tokens);
    const int col = lane & 31, hf = lane >> 5;

    // stage the codebooks of part `part` (sub-vectors part*kJP .. + kJP - 1):
    // chunk c of row (t, k) piece p -> entries (jl, c) of slice t, jl counted
    // from the part's first sub-vector
    auto stage_codebooks = [&](int part) {
        const char *src = static_cast<const char *>(cbin);
        constexpr int PER_ROW = Sh::ROWB / 16 / kParts;            // pieces of a part's row
        static_assert(PER_ROW * 16 * kParts == Sh::ROWB && (Sh::CHUNKS / kParts) % kThreads == 0,
                      "parts of whole 16-byte pieces");
#pragma unroll
        for (int u = 0; u < Sh::CHUNKS / kParts / kThreads; ++u) {
            const int c = tid + u * kThreads;
            const int r = c / PER_ROW, pc = part * PER_ROW + c % PER_ROW;
            const int t = r >> 8, k = r & 255;
            const size_t off = ((((size_t)t * a.H + h) * 256 + k) * a.S + j0) * (CG * Sh::EB) + pc * 16;
            const uint4 v = *reinterpret_cast<const uint4 *>(src + off);
            // the chunk holds runs of one sub-vector's consecutive entries
            // (a (t, k) piece of cg entries, or half of one): one aligned
            // store per run
            constexpr int RUN = CG * Sh::EB < 16 ? CG * Sh::EB : 16;   // bytes
            const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 16 / RUN; ++q) {
                const int fe = pc * Sh::EC + q * (RUN / Sh::EB);      // first element of the run
                const int jl = fe / CG - part * kJP, cc = fe % CG;
                CB *dst = cbs + (jl * 256 + k) * G + t * CG + cc;
                if constexpr (RUN == 16)
                    *reinterpret_cast<uint4 *>(dst) = v;
                else if constexpr (RUN == 8)
                    *reinterpret_cast<uint2 *>(dst) = make_uint2(vw[2 * q], vw[2 * q + 1]);
                else
                    *reinterpret_cast<uint32_t *>(dst) = vw[q];
            }
        }
    };
    constexpr int KL = Sh::KL, KC = Sh::KC, LE = Sh::LE, NLD = Sh::NLD;
    uint32_t afrag[8][NCH][KL / 2];
#pragma unroll
    for (int part = 0; part < kParts; ++part) {
        stage_codebooks(part);
        __syncthreads();
        // squared norms of the part's codes (fp64 sum, rounded once)
#pragma unroll
        for (int m = 0; m < kJP; ++m) {
            // the code's G entries as 16-byte reads (rows are 16-byte aligned)
            const uint4 *cw = reinterpret_cast<const uint4 *>(cbs + (m * 256 + tid) * G);
            double s = 0.0;
#pragma unroll
            for (int c = 0; c < G * Sh::EB / 16; ++c) {
                const uint4 w = cw[c];
                const CB *e = reinterpret_cast<const CB *>(&w);
#pragma unroll
                for (int i = 0; i < Sh::EC; ++i) {
                    const double v = to_f(e[i]);
                    s += v * v;
                }
            }
            nrm[(part * kJP + m) * 256 + tid] = (float)s;
        }
        if (wave / kJP == part) {                       // wave-uniform
            const CB *mycb = cbs + (wave - part * kJP) * 256 * G;
            // this wave's codebook as MFMA A operands: lane (col, hf) holds entries
            // kk = ch*KC + hf*KL + e of code blk*32 + col, two bf16 a word (hf enters
            // only the LDS address and the selects, so the wave builds them without
            // divergent branches)
#pragma unroll
            for (int blk = 0; blk < 8; ++blk) {
                const int code = blk * 32 + col;
                const CB *cw = mycb + code * G;
#pragma unroll
                for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
                    for (int e = 0; e < KL; e += 2) {
                        uint32_t wv = 0;
                        if constexpr (P == 1) {
                            // bf16 codebooks: -2c is a bf16 value, the upper half of
                            // the fp32 product (entries kk, kk + 1 in one word)
                            static_assert(sizeof(CB) == 2, "one part: bf16 codebooks");
                            const int kk = ch * KC + hf * KL + e;
                            const uint32_t pr = *reinterpret_cast<const uint32_t *>(cw + kk % G);
                            const uint32_t u0 = __float_as_uint(-2.f * __uint_as_float(pr << 16));
                            const uint32_t u1 = __float_as_uint(-2.f * __uint_as_float(pr & 0xffff0000u));
                            wv = kk < G ? (u0 >> 16) | (u1 & 0xffff0000u) : 0u;
                        } else {
#pragma unroll
                            for (int h2 = 0; h2 < 2; ++h2) {
                                const int kk = ch * KC + hf * KL + e + h2;
                                const float c = to_f(cw[kk % G]);
                                const float v = kk < P * G ? -2.f * split_part(c, kk / G) : 0.f;
                                wv |= (uint32_t)bf16_rne(v) << (16 * h2);
                            }
                        }
                        afrag[blk][ch][e / 2] = wv;
                    }
                }
            }
        }
        __syncthreads();                                // the part's codebooks are dead
    }
    // (S is a multiple of kJW, so every wave has a sub-vector j < S)
    float max_norm2 = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) max_norm2 = fmaxf(max_norm2, nrm[wave * 256 + lane + 64 * r]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) max_norm2 = fmaxf(max_norm2, __shfl_xor(max_norm2, off));
    // upper bound of max_k |c_k| (slack covers the rounding of the norm)
    const float max_norm = sqrtf(max_norm2) * (1.f + 1e-5f);
    // the accumulator of block blk starts at the squared norms of the lane's
    // 16 codes blk*32 + 8 q + 4 hf + i, q, i < 4 (the same for every token)
    const float *bias_row = nrm + wave * 256 + hf * 4;

    // per-lane x offsets (bytes from the tile base) of the loads that fill the
    // lane's B words: load s of chunk ch holds entries kk = ch*KC + hf*KL +
    // s*LE .. + LE - 1, i.e. x_i with i = kk mod G (step i / CG, channels
    // i mod CG ..); lanes whose K entries are not x read nothing
    uint32_t xoff[NCH][NLD];
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
        for (int s = 0; s < NLD; ++s) {
            const int kk = ch * KC + hf * KL + s * LE;
            const int i = kk % G;
            const int64_t e = (int64_t)col * a.sx_tok + (int64_t)(i / CG) * a.sx_step + (int64_t)j * CG + i % CG;
            xoff[ch][s] = kk < P * G ? (uint32_t)(2 * e) : kOob;
        }
    }

    const uint16_t *xh = xin + h * a.sx_head;
    auto rsrc = [&](int64_t n0) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(xh + n0 * a.sx_tok), (short)0,
                                                 0x7ffffff0, kBufferWord3);
    };
    uint16_t *codes = row_code[wave];
    // bit i of word t: row 32 t + i of the chunk is marked for the re-score
    uint32_t *marks = reinterpret_cast<uint32_t *>(stage + kCodeBytes) + wave * kMarkWords;

    // Tiles of 32 tokens go in groups of kDepth through two register rings:
    // while one group is screened from ring A, the next is in flight into
    // ring B, and the other way round.  A group's loads are issued a whole
    // group before its first use and after the loads of the group before it,
    // and every load of the main loop is unconditional with loop-invariant
    // lane offsets, so the compiler's wait for a group counts exactly the
    // loads behind it (a conditional load, or a per-load offset select whose
    // register gets reused for loaded data, made it wait for all of them).
    // The main loop covers whole pairs of groups; the rows after them go tile
    // by tile, where rows past the chunk's end load nothing and write no
    // code.  (A group is one tile: two fit the 128-register budget only with
    // spills, and a third ring slot, one more tile ahead, gained nothing.)
    constexpr int kTile = 32;                          // tokens per tile
    static_assert(kTokChunk / kTile == kMarkWords, "one mark word per tile");
    constexpr int kDepth = 1;                          // tiles per group
    constexpr int kPair = 2 * kTile * kDepth;          // rows of a pair of groups
    const int ntok = (int)(tok_end - tok0);
    const int nfull = ntok / kPair * kPair;
    using Tile = XTile<NCH, KL>;
    Tile ringA[kDepth], ringB[kDepth];
    // every row of the group exists (rg0 + kTile * kDepth <= nfull)
    auto load_group = [&](Tile (&rg)[kDepth], int rg0) {
#pragma unroll
        for (int u = 0; u < kDepth; ++u) load_tile<NCH, KL, LE>(rg[u], rsrc(tok0 + rg0 + kTile * u), xoff, true);
    };
    auto screen_tile = [&](const Tile &cur, const int r0) {
            const int64_t n0 = tok0 + r0;
            const bool valid = r0 + col < ntok;

            // |x|^2 from the lane's words that hold entries i < G (bf16
            // squares are exact; the sum only feeds a bound); the words are the
            // B operand as loaded
            // (with one part and G a multiple of KC every word holds entries
            // i < G, so the dot products chain through their accumulator)
            constexpr bool kAllX = P == 1 && G % KC == 0;
            float xs = 0.f;
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
                for (int q = 0; q < KL / 2; ++q) {
                    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
                    const bf16x2 v = __builtin_bit_cast(bf16x2, cur.w[ch][q]);
                    if constexpr (kAllX) {
                        xs = __builtin_amdgcn_fdot2_f32_bf16(v, v, xs, false);
                    } else {
                        const float d = __builtin_amdgcn_fdot2_f32_bf16(v, v, 0.f, false);
                        xs += (ch * KC + hf * KL + 2 * q < G) ? d : 0.f;
                    }
                }
            }
            float xa, xb;
            pair32(xs, xa, xb);
            const float xn2 = xa + xb;

            // Smallest and second smallest screen value of the lane's 128
            // codes.  The lane's value of code blk*32 + 8 (v / 4) + 4 hf + v % 4
            // (acc[v] of block blk) sits at slot s = 16 blk + v.  Two
            // partitions of the slots, groups s / 8 (half a block: acc[0..7],
            // acc[8..15]) and chains s % 8, have no two slots in common in both
            // a group and a chain, so of the two smallest values one is the
            // minimum of its group and the other the minimum of its chain or
            // of its group: the lane's second smallest is the smaller of the
            // second smallest group minimum and the second smallest chain
            // minimum.  Minima are taken with min3 over 3 operands, two new
            // values an instruction; only the 16 group and 8 chain minima get
            // marks (their low 4 bits become the group, their low 3 bits the
            // chain), and the smallest chain minimum names the chain, the
            // smallest group minimum the group of the lane's smallest value.
            // Block b + 1's MFMAs run while block b is reduced (the
            // scheduling barriers keep that order); the accumulators start at
            // the codes' squared norms, read from LDS.
            auto bias_of = [&](int blk) {
                floatx16 bv;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const floatx4 b4 = *reinterpret_cast<const floatx4 *>(bias_row + blk * 32 + 8 * q);
#pragma unroll
                    for (int i = 0; i < 4; ++i) bv[4 * q + i] = b4[i];
                }
                return bv;
            };
            auto screen = [&](int blk, floatx16 acc) {
#pragma unroll
                for (int ch = 0; ch < NCH; ++ch) acc = mfma_chunk(afrag[blk][ch], cur.w[ch], acc);
                return acc;
            };
            auto mark = [](float v, uint32_t bits, uint32_t m) {
                return __uint_as_float((__float_as_uint(v) & ~bits) | m);
            };
            auto min3 = [](float p, float q, float r) { return fminf(fminf(p, q), r); };
            floatx16 acc[2];
            acc[0] = screen(0, bias_of(0));
            acc[1] = screen(1, bias_of(1));
            __builtin_amdgcn_sched_barrier(0);
            float cm[8], g1 = 0.f, g2 = 0.f;
#pragma unroll
            for (int blk = 0; blk < 8; ++blk) {
                const floatx16 &v = acc[blk & 1];
                if constexpr (kScreen) {
                    if (valid) {
                        float *dst = a.screen + (((size_t)(n0 + col) * a.H + h) * a.S + j) * 256 + blk * 32 + 4 * hf;
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            *reinterpret_cast<float4 *>(dst + 8 * q) =
                                make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
                    }
                }
                // groups 2 blk (acc[0..7]) and 2 blk + 1 (acc[8..15])
                float ga = min3(v[0], v[1], v[2]);
                ga = min3(ga, v[3], v[4]);
                ga = min3(ga, v[5], v[6]);
                ga = mark(fminf(ga, v[7]), 15u, 2 * blk);
                float gb = min3(v[8], v[9], v[10]);
                gb = min3(gb, v[11], v[12]);
                gb = min3(gb, v[13], v[14]);
                gb = mark(fminf(gb, v[15]), 15u, 2 * blk + 1);
                // chains c (acc[c] and acc[8 + c])
                if (blk == 0) {
                    g1 = fminf(ga, gb);
                    g2 = fmaxf(ga, gb);
#pragma unroll
                    for (int c = 0; c < 8; ++c) cm[c] = fminf(v[c], v[8 + c]);
                } else {
                    g2 = fminf(g2, __builtin_amdgcn_fmed3f(g1, ga, gb));
                    g1 = min3(g1, ga, gb);
#pragma unroll
                    for (int c = 0; c < 8; ++c) cm[c] = min3(cm[c], v[c], v[8 + c]);
                }
                if (blk + 2 < 8) acc[blk & 1] = screen(blk + 2, bias_of(blk + 2));
                __builtin_amdgcn_sched_barrier(0);
            }
            // the two smallest marked chain minima
            float c1 = fminf(mark(cm[0], 7u, 0), mark(cm[1], 7u, 1));
            float c2 = fmaxf(mark(cm[0], 7u, 0), mark(cm[1], 7u, 1));
#pragma unroll
            for (int c = 2; c < 8; c += 2) {
                const float p = mark(cm[c], 7u, c), q = mark(cm[c + 1], 7u, c + 1);
                c2 = fminf(c2, __builtin_amdgcn_fmed3f(c1, p, q));
                c1 = min3(c1, p, q);
            }
            // the two lanes holding the same token combine: the lane whose
            // own smallest value is the token's smallest holds the winner
            const float own = c1;
            float m1, m2;
            {
                float a1, b1, a2, b2;
                pair32(c1, a1, b1);
                pair32(fminf(c2, g2), a2, b2);
                m2 = fminf(fmaxf(a1, b1), fminf(a2, b2));
                m1 = fminf(a1, b1);
            }
            // slot s = 8 g + c: group from the smallest group minimum, chain
            // from the smallest chain minimum
            const uint32_t slot = ((__float_as_uint(g1) & 15u) << 3) | (__float_as_uint(own) & 7u);
            const int v1 = (int)(slot & 15u);
            const int k1 = (int)(slot >> 4) * 32 + 8 * (v1 >> 2) + 4 * hf + (v1 & 3);
            const bool holder = __float_as_uint(own) == __float_as_uint(m1);
            // hardware square root (within 1 ulp): the slack covers it
            const float rad = __builtin_amdgcn_sqrtf(xn2) * (1.f + 1e-5f) + max_norm;
            const float eps = eps_scale<G, P>() * rad * rad;
            const bool unique = (m2 - m1) > eps;
            // the token's code, or the re-score mark, goes to this wave's row
            // of the LDS code array, written by one lane: the holder when the
            // winner is unique (the other lane then holds no equal value: it
            // would be the second smallest), else the lane of hf = 0
            if (valid && (unique ? holder : hf == 0)) codes[r0 + col] = unique ? (uint16_t)k1 : kRescore;
            const uint64_t mk = __ballot(valid && !unique && hf == 0);   // rows of the tile: lanes 0-31
            if (lane == 0) marks[r0 / kTile] = (uint32_t)mk;
    };
    if (nfull > 0) load_group(ringA, 0);
    for (int rb = 0; rb < nfull; rb += kPair) {
        load_group(ringB, rb + kTile * kDepth);
#pragma unroll
        for (int u = 0; u < kDepth; ++u) screen_tile(ringA[u], rb + kTile * u);
        // the last pair reloads rows of its own second group (read again,
        // never screened): the loads stay unconditional and in bounds
        load_group(ringA, rb + kPair < nfull ? rb + kPair : rb + kTile * kDepth);
#pragma unroll
        for (int u = 0; u < kDepth; ++u) screen_tile(ringB[u], rb + kTile * (kDepth + u));
    }
    for (int r0 = nfull; r0 < ntok; r0 += kTile) {
        Tile t;
        load_tile<NCH, KL, LE>(t, rsrc(tok0 + r0), xoff, r0 + col < ntok);
        screen_tile(t, r0);
    }

    // The chunk's index rows: each token's kJW codes (sub-vectors j0 ..
    // j0 + kJW - 1, one 32-bit word of its row) in one 4-byte store.  The
    // workgroups that fill the other words of these rows run alongside on the
    // same XCD, so the rows reach memory whole.
    static_assert(kMarkWords <= 64, "one mark word per lane");
    const int ntiles = (ntok + kTile - 1) / kTile;
    const uint32_t mword = lane < ntiles ? marks[lane] : 0u;   // this wave's marks
    uint64_t mtiles = __ballot(mword != 0u);
    uint8_t *out_rows = idxout + (((size_t)a.seq * a.H + h) * a.t_max + a.first_token + tok0) * a.S + j0;
    auto write_rows = [&]() {
        for (int t = tid; t < ntok; t += kThreads) {
            uint32_t w = 0;
#pragma unroll
            for (int q = 0; q < kJW; ++q) w |= (uint32_t)(row_code[q][t] & 0xffu) << (8 * q);
            *reinterpret_cast<uint32_t *>(out_rows + (size_t)t * a.S) = w;
        }
    };

    // Exact re-score of the marked rows (rare).  Every lane scores 4 codes
    // (cf[r] = code kr(r), ascending in r), then the wave takes the lowest
    // index of the smallest distance and put(row, code) records it; the mark
    // words (in registers) say which rows.
    auto rescore = [&](const float (&cf)[4][G], auto kr, auto put) {
        while (mtiles != 0) {                          // wave-uniform
            const int tt = (int)__builtin_ctzll(mtiles);
            mtiles &= mtiles - 1;
            uint32_t marked = (uint32_t)__builtin_amdgcn_readlane((int)mword, tt);
            while (marked != 0) {                      // wave-uniform
                const int rq = tt * kTile + (int)__builtin_ctz(marked);
                marked &= marked - 1;
                const uint16_t *xr = xh + (tok0 + rq) * a.sx_tok + (int64_t)j * CG;
                float xe[G];
#pragma unroll
                for (int t = 0; t < G / CG; ++t)
#pragma unroll
                    for (int c = 0; c < CG; ++c) xe[t * CG + c] = bf16f(xr[t * a.sx_step + c]);
                float best = INFINITY;
                int bk = 256;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float dist = 0.f;
#pragma unroll
                    for (int i = 0; i < G; ++i) {
                        // separate roundings: this file is built without contraction
                        const float e = xe[i] - cf[r][i];
                        const float sq = e * e;
                        dist = dist + sq;
                    }
                    if (dist < best) {
                        best = dist;
                        bk = kr(r);
                    }
                }
                // distances are >= 0, so their bit patterns order like them
                const uint32_t dmin = wave_min_u32(__float_as_uint(best));
                const uint32_t kmin = wave_min_u32(__float_as_uint(best) == dmin ? (uint32_t)bk : 256u);
                put(rq, kmin);
            }
        }
    };
    if constexpr (P == 1) {
        // bf16 codebooks: the wave's MFMA operands still hold -2c (exact) for
        // all 256 codes, lane (col, hf) entries kk = ch*KC + hf*KL + e of
        // codes 32 blk + col.  One lane swap per operand word pairs blocks b
        // and b + 4: afterwards lane (col, hf) holds every entry of code
        // 32 (b + 4 hf) + col (its first KL of each K chunk in the first
        // result, the next KL in the second), so no codebook is read again.
        // c = -0.5 (-2c) is exact.  The exact code replaces the mark in the
        // wave's row of the LDS code array, so each row is written once.
        if (mtiles != 0) {                             // wave-uniform
            float cf[4][G];
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
                    for (int w = 0; w < KL / 2; ++w) {
                        const auto r = __builtin_amdgcn_permlane32_swap(afrag[b][ch][w], afrag[b + 4][ch][w],
                                                                        false, false);
#pragma unroll
                        for (int q = 0; q < 2; ++q)
#pragma unroll
                            for (int h2 = 0; h2 < 2; ++h2) {
                                const int i = ch * KC + q * KL + 2 * w + h2;
                                const uint32_t word = q ? r[1] : r[0];
                                if (i < G)
                                    cf[b][i] = -0.5f * __uint_as_float(h2 ? (word & 0xffff0000u) : (word << 16));
                            }
                    }
            rescore(cf, [&](int r) { return 32 * (r + 4 * hf) + col; },
                    [&](int rq, uint32_t k) {
                        if (lane == 0) codes[rq] = (uint16_t)k;
                    });
        }
        __syncthreads();
        write_rows();
    } else {
        __syncthreads();
        write_rows();                                  // marked rows hold a placeholder byte
        // (the words are written before any re-scored byte of them: the
        // barrier also waits for the stores)
        __syncthreads();
        // fp32 codebooks (three bf16 parts in the operands): the code array
        // is dead, so the workgroup stages its codebooks in LDS again (one
        // coalesced pass for the 4 sub-vectors) and lane l takes codes
        // l + 64 r from there; the re-scored byte replaces the placeholder.
        if (__syncthreads_or(mtiles != 0)) {           // workgroup-uniform
            stage_codebooks(0);
            __syncthreads();
            if (mtiles != 0) {                         // wave-uniform
                float cf[4][G];
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int i = 0; i < G; ++i) cf[r][i] = to_f(cbs[(wave * 256 + lane + 64 * r) * G + i]);
                rescore(cf, [&](int r) { return lane + 64 * r; },
                        [&](int rq, uint32_t k) {
                            if (lane == 0) out_rows[(size_t)rq * a.S + wave] = (uint8_t)k;
                        });
            }
        }
    }
}

// Direct path for short runs (a page of generated tokens, up to kSmallTokens).
// A workgroup takes kJW adjacent sub-vectors j of one head h and all 256
// codes: lane (c, jj) of wave w (c = lane % 16, jj = lane / 16) scores codes
// k = (16 w + c) R + r, r < R, for sub-vector j0 + jj, so the 16 lanes of a
// row share one sub-vector and each code row is read as kJW adjacent slice
// entries (one contiguous piece of a cache line, not one entry per line).
// Every distance is evaluated exactly as defined; a lane keeps its lowest
// code of the smallest distance (strict < in ascending k), the row takes the
// smallest distance (distances are >= 0, so their bit patterns order like
// them) and then the lowest code holding it, and the lowest wave (lowest
// codes) wins ties across waves.  No screen, so nothing is re-scored.
constexpr int kSmallTokens = 32;
constexpr int kSmallThreads = 1024;

template <int CG, typename CB>
__device__ __forceinline__ void load_entries(const CB *src, float *out) {
    constexpr int NB = CG * (int)sizeof(CB);           // bytes of one slice entry
    uint32_t w[NB / 4];
    if constexpr (NB >= 16) {
#pragma unroll
        for (int q = 0; q < NB / 16; ++q) {
            const uint4 v = reinterpret_cast<const uint4 *>(src)[q];
            w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
        }
    } else if constexpr (NB == 8) {
        const uint2 v = *reinterpret_cast<const uint2 *>(src);
        w[0] = v.x; w[1] = v.y;
    } else {
        w[0] = *reinterpret_cast<const uint32_t *>(src);
    }
#pragma unroll
    for (int c = 0; c < CG; ++c) {
        if constexpr (sizeof(CB) == 2)
            out[c] = __uint_as_float((c & 1) ? (w[c >> 1] & 0xffff0000u) : (w[c >> 1] << 16));
        else
            out[c] = __uint_as_float(w[c]);
    }
}

// minimum over the 16 lanes of a row, in every lane of it (DPP only)
__device__ __forceinline__ uint32_t row_min_u32(uint32_t v) {
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, false));  // row_ror 8
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xf, 0xf, false));  // row_ror 4
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, false));   // xor 2
    return min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false)); // xor 1
}

template <int G, int CG, typename CB>
__global__ __launch_bounds__(kSmallThreads) void encode_small(EncodeArgs a) {
    constexpr int NW = kSmallThreads / 64;
    constexpr int R = 256 / (NW * 16);                 // codes per lane
    constexpr int XR = G + 4;                          // padded row: conflict-free 16-B reads
    __shared__ __align__(16) float xs[kSmallTokens][kJW][XR];
    __shared__ uint32_t wave_d[NW][kSmallTokens][kJW], wave_k[NW][kSmallTokens][kJW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane & 15, jj = lane >> 4;
    // the workgroups of one (head, tensor) read the same code rows: keep them
    // on one XCD (workgroups are dealt to the 8 XCDs in turn)
    const int nj = a.S / kJW;
    const int n_wg = nj * a.H * a.n_tensors;
    int L = blockIdx.x;
    if (n_wg % 8 == 0) L = (L % 8) * (n_wg / 8) + L / 8;
    const int jb = L % nj, h = (L / nj) % a.H, z = L / (nj * a.H);
    const int j0 = jb * kJW;
    const uint16_t *xin = z ? a.x_b : a.x;
    uint8_t *idxout = z ? a.index_b : a.index;
    const int n = (int)a.n_tokens;
    for (int e = tid; e < n * kJW * G; e += kSmallThreads) {
        const int tok = e / (kJW * G), q = (e / G) % kJW, i = e % G;
        xs[tok][q][i] = bf16f(xin[tok * a.sx_tok + h * a.sx_head + (i / CG) * a.sx_step +
                                  (int64_t)(j0 + q) * CG + i % CG]);
    }
    const CB *cb = static_cast<const CB *>(z ? a.cb_b : a.cb);
    const int k0 = (wave * 16 + c) * R;
    float cw[R][G];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < G / CG; ++t)
            load_entries<CG, CB>(cb + ((((size_t)t * a.H + h) * 256 + k0 + r) * a.S + j0 + jj) * CG,
                                 &cw[r][t * CG]);
    __syncthreads();
    for (int t0 = 0; t0 < n; t0 += 4) {
        uint32_t best[4], bk[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int tok = min(t0 + q, n - 1);
            float xv[G];
#pragma unroll
            for (int i = 0; i < G; i += 4) {
                const float4 v = *reinterpret_cast<const float4 *>(&xs[tok][jj][i]);
                xv[i] = v.x; xv[i + 1] = v.y; xv[i + 2] = v.z; xv[i + 3] = v.w;
            }
            best[q] = 0xffffffffu;
            bk[q] = 0;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float dd = 0.f;
#pragma unroll
                for (int i = 0; i < G; ++i) {
                    const float e = xv[i] - cw[r][i];
                    const float sq = e * e;
                    dd = dd + sq;
                }
                if (__float_as_uint(dd) < best[q]) {
                    best[q] = __float_as_uint(dd);
                    bk[q] = k0 + r;
                }
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t dmin = row_min_u32(best[q]);
            const uint32_t kmin = row_min_u32(best[q] == dmin ? bk[q] : 256u);
            if (c == 0 && t0 + q < n) {
                wave_d[wave][t0 + q][jj] = dmin;
                wave_k[wave][t0 + q][jj] = kmin;
            }
        }
    }
    __syncthreads();
    if (tid < n * kJW) {
        const int tok = tid / kJW, q = tid % kJW;
        uint32_t bd = wave_d[0][tok][q], bkk = wave_k[0][tok][q];
#pragma unroll
        for (int w = 1; w < NW; ++w) {
            if (wave_d[w][tok][q] < bd) {
                bd = wave_d[w][tok][q];
                bkk = wave_k[w][tok][q];
            }
        }
        idxout[(((size_t)a.seq * a.H + h) * a.t_max + a.first_token + tok) * a.S + j0 + q] = (uint8_t)bkk;
    }
}

// workgroups of encode_kernel: token chunks x groups of kJW sub-vectors x
// heads x tensors (one linear grid)
inline unsigned screen_workgroups(const EncodeArgs &a) {
    return (unsigned)(((a.n_tokens + kTokChunk - 1) / kTokChunk) * ((a.S + kJW - 1) / kJW) * a.H * a.n_tensors);
}

template <int G, int CG>
hipError_t launch_gc(const EncodeArgs &a, hipStream_t st) {
    if (a.screen) {
        // the screen path at any length, storing the screen values
        const dim3 grid(screen_workgroups(a));
        if (a.cb_bf16)
            hipLaunchKernelGGL((encode_kernel<G, CG, 1, uint16_t, true>), grid, dim3(kThreads), 0, st, a);
        else if constexpr (G <= 16)
            hipLaunchKernelGGL((encode_kernel<G, CG, 3, float, true>), grid, dim3(kThreads), 0, st, a);
        else
            return hipErrorInvalidValue;
        return hipGetLastError();
    }
    if (a.n_tokens <= kSmallTokens) {
        const dim3 grid((unsigned)(a.S / kJW * a.H * a.n_tensors));
        if (a.cb_bf16)
            hipLaunchKernelGGL((encode_small<G, CG, uint16_t>), grid, dim3(kSmallThreads), 0, st, a);
        else if constexpr (G <= 16)
            hipLaunchKernelGGL((encode_small<G, CG, float>), grid, dim3(kSmallThreads), 0, st, a);
        else
            return hipErrorInvalidValue;
        return hipGetLastError();
    }
    const dim3 grid(screen_workgroups(a));
    if (a.cb_bf16) {
        hipLaunchKernelGGL((encode_kernel<G, CG, 1, uint16_t, false>), grid, dim3(kThreads), 0, st, a);
    } else {
        if constexpr (G <= 16)
            hipLaunchKernelGGL((encode_kernel<G, CG, 3, float, false>), grid, dim3(kThreads), 0, st, a);
        else
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

bool encode_supported(int G, int cg, int S, int cb_bf16) {
    if (G != 8 && G != 16 && G != 32) return false;
    if (cg != 2 && cg != 4 && cg != 8) return false;
    if (cg > G) return false;
    if (S % kJW != 0) return false;                    // whole workgroups of sub-vectors
    if (!cb_bf16 && G > 16) return false;
    return true;
}

hipError_t launch_encode(const EncodeArgs &a, hipStream_t st) {
#define LVQ_CASE(G_, CG_) \
    if (a.G == G_ && a.cg == CG_) return launch_gc<G_, CG_>(a, st);
    LVQ_CASE(8, 2)
    LVQ_CASE(8, 4)
    LVQ_CASE(8, 8)
    LVQ_CASE(16, 2)
    LVQ_CASE(16, 4)
    LVQ_CASE(16, 8)
    LVQ_CASE(32, 2)
    LVQ_CASE(32, 4)
    LVQ_CASE(32, 8)
#undef LVQ_CASE
    return hipErrorInvalidValue;
}

}  // namespace lvq
