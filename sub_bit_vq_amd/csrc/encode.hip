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
// piece is one contiguous read) in LDS, with their squared norms.
//
// Screen (MFMA).  The screen value S_k = |c_k|^2 - 2 x.c_k differs from D_k by
// |x|^2, the same for every k.  One v_mfma_f32_16x16x32_bf16 multiplies 16
// codes (rows) by 16 tokens (columns) over an augmented K axis:
//     code row  = [-2 c_k (split into P bf16 parts), b0, b1, b2, 0...]
//     token col = [ x (repeated P times),           1,  1,  1, 0...]
// where b0 + b1 + b2 = fl32(|c_k|^2) in bf16 parts (and, for fp32 codebooks,
// c = c0 + c1 + c2 in bf16 parts, P = 3).  Products of bf16 values are exact
// in fp32, so the only screen errors are the accumulation roundings.  Each
// wave keeps its codebook in registers as MFMA A operands and streams 16-token
// tiles through it.  Each lane tracks the two smallest screen values of its 64
// codes, a pair (a, b) at a time: the smallest is min3(m1, a, b) and the
// second smallest min(m2, med3(m1, a, b)).  The low 6 bits of each value are
// replaced by its slot among the lane's 64 codes, so the smallest value also
// names its code (the lane supplies the rest of the index).
//
// Exactness.  With R = |x| + max_k |c_k|, the 6 bits written into a value
// move it by at most 2^-17 R^2; the fp32 error of D_k is at most
// (G+2) 2^-24 R^2 and that of the screen at most F (P*G+3) 2^-24 R^2 for an
// accumulation F times worse than a sequential fp32 sum.  If the two smallest
// (marked) screen values are more than eps = 2^-14 R^2 apart, eps exceeds
// twice the sum of these (for F up to 10 at G = 32, P = 1 and up to 7 at
// G = 16, P = 3), so the screen
// winner is the exact winner.  Otherwise the wave re-scores all 256 codes of
// that sub-vector exactly as defined above from the staged codebook (64 lanes
// x 4 codes, strict < per lane in ascending k, then a lowest-index argmin
// across lanes), which reproduces the definition bit for bit.
#include "kernels.h"

#include <math.h>

#pragma clang fp contract(off)

namespace lvq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;     // 4 waves, one sub-vector index j each
constexpr int kJW = 4;            // sub-vectors per workgroup
constexpr int kTokChunk = 2048;   // tokens per workgroup (queued rows fit 16 bits)
constexpr float kEpsScale = 6.103515625e-05f;  // 2^-14

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
    static constexpr int KAUG = (P * G + 3 + 31) / 32 * 32;
    static constexpr int NCH = KAUG / 32;                  // MFMAs per 16 codes x 16 tokens
    static constexpr int EB = (int)sizeof(CB);
    static constexpr int ROWB = kJW * CG * EB;             // bytes of one (slice, code) row piece
    static constexpr int EC = 16 / EB;                     // elements per 16-byte chunk
    static constexpr int CHUNKS = T * 256 * ROWB / 16;     // staging chunks
    static_assert(ROWB % 16 == 0 && CHUNKS % kThreads == 0, "staging tiles");
    static_assert(G % 8 == 0 && (P * G) % 8 == 0, "operand blocks of 8");
};

// One 16-token tile of x as MFMA B-operand words: lane (row, kq) holds, for
// each K chunk ch, the 4 words (8 bf16) of entries kk = ch*32 + kq*8 .. +7 of
// token n0 + row (zero where kk is not an x entry or the token is past the end).
template <int NCH>
struct XTile {
    uint32_t w[NCH][4];
};

constexpr uint32_t kOob = 0xffffff00u;            // offset past any buffer: loads return 0
constexpr int kBufferWord3 = 0x00020000;          // raw buffer resource, gfx9 family

template <int CG, int NCH>
__device__ __forceinline__ void load_tile(XTile<NCH> &t, __amdgpu_buffer_rsrc_t rs,
                                          const uint32_t (&off)[NCH][8 / CG > 0 ? 8 / CG : 1],
                                          bool valid) {
    constexpr int NLD = 8 / CG;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
        for (int s = 0; s < NLD; ++s) {
            const uint32_t o = valid ? off[ch][s] : kOob;
            if constexpr (CG == 8) {
                const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, 0));
                t.w[ch][0] = v.x; t.w[ch][1] = v.y; t.w[ch][2] = v.z; t.w[ch][3] = v.w;
            } else if constexpr (CG == 4) {
                const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, o, 0, 0));
                t.w[ch][2 * s] = v.x; t.w[ch][2 * s + 1] = v.y;
            } else {
                t.w[ch][s] = __builtin_amdgcn_raw_buffer_load_b32(rs, o, 0, 0);
            }
        }
    }
}

template <int G, int CG, int P, typename CB>
__global__ __launch_bounds__(kThreads) void encode_kernel(EncodeArgs a) {
    using Sh = EncShape<G, CG, P, CB>;
    constexpr int NCH = Sh::NCH;
    __shared__ __align__(16) CB cbs[kJW * 256 * G];    // [jl][k][i]
    __shared__ float nrm[kJW * 256];
    __shared__ uint16_t amb_queue[kJW][kTokChunk];     // per wave: chunk rows to re-score
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // grid z = tensor * H + head (a launch may encode two tensors, e.g. K and V)
    const int tz = (int)blockIdx.z / a.H;
    const int h = (int)blockIdx.z - tz * a.H;
    const uint16_t *xin = tz ? a.x_b : a.x;
    const void *cbin = tz ? a.cb_b : a.cb;
    uint8_t *idxout = tz ? a.index_b : a.index;
    const int j0 = blockIdx.y * kJW, j = j0 + wave;
    const int64_t tok0 = (int64_t)blockIdx.x * kTokChunk;
    const int64_t tok_end = min(tok0 + kTokChunk, a.n_tokens);
    const int row = lane & 15, kq = lane >> 4;

    // stage the 4 codebooks: chunk c of row (t, k) piece p -> entries (jl, c) of slice t
    {
        const char *src = static_cast<const char *>(cbin);
        constexpr int PER_ROW = Sh::ROWB / 16;
#pragma unroll
        for (int u = 0; u < Sh::CHUNKS / kThreads; ++u) {
            const int c = tid + u * kThreads;
            const int r = c / PER_ROW, pc = c % PER_ROW;
            const int t = r >> 8, k = r & 255;
            const size_t off = ((((size_t)t * a.H + h) * 256 + k) * a.S + j0) * (CG * Sh::EB) + pc * 16;
            const uint4 v = *reinterpret_cast<const uint4 *>(src + off);
            const CB *e = reinterpret_cast<const CB *>(&v);
#pragma unroll
            for (int q = 0; q < Sh::EC; ++q) {
                const int fe = pc * Sh::EC + q;          // element of the (t, k) row piece
                const int jl = fe / CG, cc = fe % CG;
                cbs[(jl * 256 + k) * G + t * CG + cc] = e[q];
            }
        }
    }
    __syncthreads();
    // squared norms (fp64 sum, rounded once); the max over the wave's codes
#pragma unroll
    for (int m = 0; m < kJW; ++m) {
        const CB *cw = cbs + (m * 256 + tid) * G;
        double s = 0.0;
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const double v = to_f(cw[i]);
            s += v * v;
        }
        nrm[m * 256 + tid] = (float)s;
    }
    __syncthreads();
    if (j >= a.S) return;
    float max_norm2 = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) max_norm2 = fmaxf(max_norm2, nrm[wave * 256 + lane + 64 * r]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) max_norm2 = fmaxf(max_norm2, __shfl_xor(max_norm2, off));
    // upper bound of max_k |c_k| (slack covers the rounding of the norm)
    const float max_norm = sqrtf(max_norm2) * (1.f + 1e-5f);

    // this wave's codebook as MFMA A operands: lane (row, kq) holds entries
    // kk = ch*32 + kq*8 + e of code blk*16 + row (kq unrolled so that every
    // register index is a constant)
    const CB *mycb = cbs + wave * 256 * G;
    bf16x8 afrag[16][NCH];
#pragma unroll
    for (int blk = 0; blk < 16; ++blk) {
        const int code = blk * 16 + row;
        const CB *cw = mycb + code * G;
        const float bias = nrm[wave * 256 + code];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (kq != q) continue;
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) {
                bf16x8 f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int kk = ch * 32 + q * 8 + e;
                    float v = 0.f;
                    if (kk < P * G)
                        v = -2.f * (P == 1 ? to_f(cw[kk % G]) : split_part(to_f(cw[kk % G]), kk / G));
                    else if (kk < P * G + 3)
                        v = split_part(bias, kk - P * G);
                    f[e] = __builtin_bit_cast(__bf16, bf16_rne(v));
                }
                afrag[blk][ch] = f;
            }
        }
    }

    uint8_t *out_rows = idxout + (((size_t)a.seq * a.H + h) * a.t_max + a.first_token) * a.S + j;

    // per-lane x offsets (bytes from the tile base) of the loads that fill the
    // lane's B words; lanes whose K entries are not x read nothing
    constexpr int NLD = 8 / CG;
    uint32_t xoff[NCH][NLD];
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        const int kk0 = ch * 32 + kq * 8;
        const int i0 = kk0 % G;
#pragma unroll
        for (int s = 0; s < NLD; ++s) {
            const int64_t e = (int64_t)row * a.sx_tok + (int64_t)(i0 / CG + s) * a.sx_step +
                              (int64_t)j * CG;
            xoff[ch][s] = kk0 < P * G ? (uint32_t)(2 * e) : kOob;
        }
    }
    // the three ones of the bias column sit in the K chunk and lanes of kk = P*G
    constexpr int ONES_CH = P * G / 32;
    const bool ones_lane = kq == (P * G % 32) / 8;
    const uint32_t ones0 = ones_lane ? 0x3f803f80u : 0u;    // bf16 1.0, 1.0
    const uint32_t ones1 = ones_lane ? 0x00003f80u : 0u;    // bf16 1.0, 0
    // lanes whose words are x entries i < G (counted once for |x|^2)
    const bool norm_lane = kq * 8 < G;

    const uint16_t *xh = xin + h * a.sx_head;
    auto rsrc = [&](int64_t n0) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(xh + n0 * a.sx_tok), (short)0,
                                                 0x7ffffff0, kBufferWord3);
    };
    uint16_t *queue = amb_queue[wave];
    int n_amb = 0;

    // tiles are processed in groups of kDepth; rows past the chunk's end (a
    // ragged last group) load nothing and store nothing
    constexpr int kDepth = 4;                          // tiles in flight per wave
    const int ntok = (int)(tok_end - tok0);
    XTile<NCH> ring[kDepth];
#pragma unroll
    for (int u = 0; u < kDepth; ++u)
        load_tile<CG, NCH>(ring[u], rsrc(tok0 + 16 * u), xoff, 16 * u + row < ntok);

    for (int rb = 0; rb < ntok; rb += 16 * kDepth) {
#pragma unroll
        for (int u = 0; u < kDepth; ++u) {
            const int r0 = rb + 16 * u;                // tile's first row in the chunk
            const int64_t n0 = tok0 + r0;
            const XTile<NCH> cur = ring[u];
            {
                const int rn = r0 + 16 * kDepth;
                load_tile<CG, NCH>(ring[u], rsrc(tok0 + rn), xoff, rn + row < ntok);
            }
            const bool valid = r0 + row < ntok;

            // B operand and |x|^2 (bf16 squares are exact; the sum only feeds a bound)
            bf16x8 bfrag[NCH];
            float xs = 0.f;
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) {
                uint32_t w0 = cur.w[ch][0], w1 = cur.w[ch][1];
                if (ch == 0) {
                    float d = 0.f;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
                        const bf16x2 v = __builtin_bit_cast(bf16x2, cur.w[0][q]);
                        d = __builtin_amdgcn_fdot2_f32_bf16(v, v, d, false);
                    }
                    xs = norm_lane ? d : 0.f;
                }
                if (ch == ONES_CH) {
                    w0 |= ones0;
                    w1 |= ones1;
                }
                bfrag[ch] = __builtin_bit_cast(bf16x8, make_uint4(w0, w1, cur.w[ch][2], cur.w[ch][3]));
            }
            float xa, xb;
            pair16(xs, xa, xb);
            pair32(xa + xb, xa, xb);
            const float xn2 = xa + xb;

            // two smallest marked screen values of the lane's 64 codes, taken a
            // pair (a, b) at a time: with m1 <= m2, the second smallest of
            // {m1, m2, a, b} is min(m2, med3(m1, a, b)) and the smallest is
            // min3(m1, a, b)
            // MFMAs run kPipe blocks ahead of the min tracking so that their
            // latency overlaps it (the scheduling barriers keep that order)
            constexpr int kPipe = 4;
            auto screen = [&](int blk) {
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ch = 0; ch < NCH; ++ch)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag[blk][ch], bfrag[ch], acc, 0, 0, 0);
                return acc;
            };
            floatx4 accs[kPipe];
#pragma unroll
            for (int p = 0; p < kPipe; ++p) accs[p] = screen(p);
            __builtin_amdgcn_sched_barrier(0);
            float m1 = INFINITY, m2 = INFINITY;
#pragma unroll
            for (int blk = 0; blk < 16; ++blk) {
                const floatx4 acc = accs[blk % kPipe];
                // lane holds codes blk*16 + kq*4 + i of token n0 + row; the low
                // 6 bits of each value become its slot blk*4 + i in the lane
                float v[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    v[i] = __uint_as_float((__float_as_uint(acc[i]) & 0xffffffc0u) | (uint32_t)(blk * 4 + i));
#pragma unroll
                for (int i = 0; i < 4; i += 2) {
                    m2 = fminf(m2, __builtin_amdgcn_fmed3f(m1, v[i], v[i + 1]));
                    m1 = fminf(m1, fminf(v[i], v[i + 1]));
                }
                if (blk + kPipe < 16) accs[blk % kPipe] = screen(blk + kPipe);
                __builtin_amdgcn_sched_barrier(0);
            }
            // combine the four lanes holding the same token; the lane whose own
            // smallest value is the token's smallest holds the winner
            const float own = m1;
            {
                float a1, b1, a2, b2;
                pair16(m1, a1, b1);
                pair16(m2, a2, b2);
                m2 = fminf(fmaxf(a1, b1), fminf(a2, b2));
                m1 = fminf(a1, b1);
                pair32(m1, a1, b1);
                pair32(m2, a2, b2);
                m2 = fminf(fmaxf(a1, b1), fminf(a2, b2));
                m1 = fminf(a1, b1);
            }
            const uint32_t slot = __float_as_uint(m1) & 63u;
            const int k1 = (int)((slot >> 2) * 16 + kq * 4 + (slot & 3));
            const bool holder = __float_as_uint(own) == __float_as_uint(m1);
            // hardware square root (within 1 ulp): the slack covers it
            const float rad = __builtin_amdgcn_sqrtf(xn2) * (1.f + 1e-5f) + max_norm;
            const float eps = kEpsScale * rad * rad;
            const bool unique = (m2 - m1) > eps;
            // when the winner is unique no other lane holds an equal value (it
            // would be the second smallest), so exactly one lane stores
            if (holder && valid && unique) out_rows[(size_t)(n0 + row) * a.S] = (uint8_t)k1;

            // queue the ambiguous sub-vectors of this tile (rows of the chunk)
            const bool amb = kq == 0 && valid && !unique;
            const uint64_t amb_mask = __ballot(amb);
            if (amb) {
                const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(amb_mask >> 32),
                                                          __builtin_amdgcn_mbcnt_lo((uint32_t)amb_mask, 0));
                queue[n_amb + pos] = (uint16_t)(r0 + row);
            }
            n_amb += __builtin_popcountll(amb_mask);
        }
    }

    // exact re-score of the queued sub-vectors: every lane scores 4 codes
    // k = lane + 64 r, then the wave takes the lowest index of the smallest
    // distance
    float cf[4][G];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < G; ++i) cf[r][i] = to_f(mycb[(lane + 64 * r) * G + i]);
    for (int q = 0; q < n_amb; ++q) {
        const int rq = __builtin_amdgcn_readfirstlane(queue[q]);
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
                bk = lane + 64 * r;
            }
        }
        // distances are >= 0, so their bit patterns order like them
        const uint32_t dmin = wave_min_u32(__float_as_uint(best));
        const uint32_t kmin = wave_min_u32(__float_as_uint(best) == dmin ? (uint32_t)bk : 256u);
        if (lane == 0) out_rows[(size_t)(tok0 + rq) * a.S] = (uint8_t)kmin;
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

template <int G, int CG>
hipError_t launch_gc(const EncodeArgs &a, hipStream_t st) {
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
    const dim3 grid((unsigned)((a.n_tokens + kTokChunk - 1) / kTokChunk), (a.S + kJW - 1) / kJW,
                    a.H * a.n_tensors);
    if (a.cb_bf16) {
        hipLaunchKernelGGL((encode_kernel<G, CG, 1, uint16_t>), grid, dim3(kThreads), 0, st, a);
    } else {
        if constexpr (G <= 16)
            hipLaunchKernelGGL((encode_kernel<G, CG, 3, float>), grid, dim3(kThreads), 0, st, a);
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
