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
// Screen (MFMA).  The screen value S_k = |c_k|^2 - 2 x.c_k differs from D_k by
// |x|^2, the same for every k.  One v_mfma_f32_16x16x32_bf16 multiplies 16
// codes (rows) by 16 tokens (columns) over an augmented K axis:
//     code row  = [-2 c_k (split into P bf16 parts), b0, b1, b2, 0...]
//     token col = [ x (repeated P times),           1,  1,  1, 0...]
// where b0 + b1 + b2 = fl32(|c_k|^2) in bf16 parts (and, for fp32 codebooks,
// c = c0 + c1 + c2 in bf16 parts, P = 3).  Products of bf16 values are exact
// in fp32, so the only screen errors are the accumulation roundings.  Each
// wave keeps its (h, j) codebook resident in registers as MFMA A operands and
// streams 16-token tiles through it; every lane tracks the smallest and
// second-smallest screen value of its 64 codes, and 4 lanes combine.
//
// Exactness.  If the two smallest screen values are more than
//     eps = 2^-14 (|x| + max_k |c_k|)^2
// apart, the screen winner is the exact winner: eps exceeds twice the sum of
// the fp32 error of D_k (at most (G+2) 2^-24 D_k) and of the screen (at most
// F (P*G+3) 2^-24 (|c|^2 + 2|x||c|) for an accumulation F times worse than a
// sequential fp32 sum), for F up to 13 at G = 32 and P = 1.  Otherwise the
// wave re-scores all 256 codes of that sub-vector exactly as defined above (64
// lanes x 4 codes, strict < per lane in ascending k, then a lowest-index
// argmin across lanes), which reproduces the definition bit for bit.
#include "kernels.h"

#include <math.h>

#pragma clang fp contract(off)

namespace lvq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;     // 4 waves, one sub-vector index j each
constexpr int kTokChunk = 1024;   // tokens per workgroup
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
__device__ __forceinline__ float cb_at(const CB *p, size_t i);
template <>
__device__ __forceinline__ float cb_at<float>(const float *p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float cb_at<uint16_t>(const uint16_t *p, size_t i) { return bf16f(p[i]); }

// entry i = t*CG + c of codeword k of (h, j): codebook [Tc][H][256][S][CG]
template <int CG, typename CB>
__device__ __forceinline__ float codeword(const EncodeArgs &a, const CB *cb, int h, int j, int k,
                                          int i) {
    const int t = i / CG, c = i % CG;
    return cb_at(cb, ((((size_t)t * a.H + h) * 256 + k) * a.S + j) * CG + c);
}

// sub-vector entries x_0..x_{G-1} of (token n, head h, sub-vector j)
template <int G, int CG>
__device__ __forceinline__ void load_subvector(const EncodeArgs &a, int64_t n, int h, int j,
                                               float (&xv)[G]) {
    const uint16_t *base = a.x + n * a.sx_tok + h * a.sx_head + (int64_t)j * CG;
#pragma unroll
    for (int t = 0; t < G / CG; ++t) {
        const uint16_t *p = base + t * a.sx_step;
        if constexpr (CG == 8) {
            const uint4 v = *reinterpret_cast<const uint4 *>(p);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xv[t * 8 + 2 * e] = __uint_as_float(w[e] << 16);
                xv[t * 8 + 2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
            }
        } else if constexpr (CG == 4) {
            const uint2 v = *reinterpret_cast<const uint2 *>(p);
            xv[t * 4 + 0] = __uint_as_float(v.x << 16);
            xv[t * 4 + 1] = __uint_as_float(v.x & 0xffff0000u);
            xv[t * 4 + 2] = __uint_as_float(v.y << 16);
            xv[t * 4 + 3] = __uint_as_float(v.y & 0xffff0000u);
        } else {
            const uint32_t v = *reinterpret_cast<const uint32_t *>(p);
            xv[t * 2 + 0] = __uint_as_float(v << 16);
            xv[t * 2 + 1] = __uint_as_float(v & 0xffff0000u);
        }
    }
}

// D_k exactly as defined: sequential fp32, no contraction.
template <int G, int CG, typename CB>
__device__ __forceinline__ float exact_distance(const EncodeArgs &a, const CB *cb, int h, int j,
                                                int k, const float (&xv)[G]) {
    float dist = 0.f;
#pragma unroll
    for (int i = 0; i < G; ++i) {
        const float e = __fsub_rn(xv[i], codeword<CG>(a, cb, h, j, k, i));
        dist = __fadd_rn(dist, __fmul_rn(e, e));
    }
    return dist;
}

template <int G, int CG, int P, typename CB>
__global__ __launch_bounds__(kThreads) void encode_kernel(EncodeArgs a) {
    constexpr int KAUG = (P * G + 3 + 31) / 32 * 32;
    constexpr int NCH = KAUG / 32;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = blockIdx.z;
    const int j = blockIdx.y * 4 + wave;
    if (j >= a.S) return;
    const int64_t tok0 = (int64_t)blockIdx.x * kTokChunk;
    const int64_t tok_end = min(tok0 + kTokChunk, a.n_tokens);
    const CB *cb = static_cast<const CB *>(a.cb);
    const int row = lane & 15, kq = lane >> 4;

    // codebook of (h, j) as MFMA A operands; max codeword norm
    bf16x8 afrag[16][NCH];
    float max_norm2 = 0.f;
#pragma unroll
    for (int blk = 0; blk < 16; ++blk) {
        const int code = blk * 16 + row;
        float cw[G];
        double n2 = 0.0;
#pragma unroll
        for (int i = 0; i < G; ++i) {
            cw[i] = codeword<CG>(a, cb, h, j, code, i);
            n2 += (double)cw[i] * (double)cw[i];
        }
        const float bias = (float)n2;
        max_norm2 = fmaxf(max_norm2, bias);
        // augmented row entries kk = ch*32 + kq*8 + e; the lane-group index
        // kq is unrolled so that every register index is a constant
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
                        v = -2.f * (P == 1 ? cw[kk % G] : split_part(cw[kk % G], kk / G));
                    else if (kk < P * G + 3)
                        v = split_part(bias, kk - P * G);
                    f[e] = __builtin_bit_cast(__bf16, bf16_rne(v));
                }
                afrag[blk][ch] = f;
            }
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) max_norm2 = fmaxf(max_norm2, __shfl_xor(max_norm2, off));
    // upper bound of max_k |c_k| (slack covers the rounding of the norm)
    const float max_norm = sqrtf(max_norm2) * (1.f + 1e-5f);

    uint8_t *out_rows = a.index + (((size_t)a.seq * a.H + h) * a.t_max + a.first_token) * a.S + j;

    for (int64_t n0 = tok0; n0 < tok_end; n0 += 16) {
        const int64_t n = n0 + row;
        const bool valid = n < tok_end;
        float xv[G];
        if (valid) {
            load_subvector<G, CG>(a, n, h, j, xv);
        } else {
#pragma unroll
            for (int i = 0; i < G; ++i) xv[i] = 0.f;
        }
        float xn2 = 0.f;
#pragma unroll
        for (int i = 0; i < G; ++i) xn2 += xv[i] * xv[i];

        bf16x8 bfrag[NCH];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (kq != q) continue;
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int kk = ch * 32 + q * 8 + e;
                    float v = 0.f;
                    if (kk < P * G)
                        v = xv[kk % G];
                    else if (kk < P * G + 3)
                        v = 1.f;
                    bfrag[ch][e] = __builtin_bit_cast(__bf16, bf16_rne(v));
                }
            }
        }

        float m1 = INFINITY, m2 = INFINITY;
        int k1 = 0;
#pragma unroll
        for (int blk = 0; blk < 16; ++blk) {
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag[blk][ch], bfrag[ch], acc, 0, 0, 0);
            // lane holds codes blk*16 + kq*4 + i of token n0 + row
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v = acc[i];
                if (v < m1) {
                    m2 = m1;
                    m1 = v;
                    k1 = blk * 16 + kq * 4 + i;
                } else {
                    m2 = fminf(m2, v);
                }
            }
        }
        // combine the four lanes holding the same token
#pragma unroll
        for (int off = 16; off <= 32; off <<= 1) {
            const float om1 = __shfl_xor(m1, off);
            const float om2 = __shfl_xor(m2, off);
            const int ok1 = __shfl_xor(k1, off);
            const float nm2 = fminf(fminf(m2, om2), fmaxf(m1, om1));
            if (om1 < m1 || (om1 == m1 && ok1 < k1)) {
                m1 = om1;
                k1 = ok1;
            }
            m2 = nm2;
        }
        const float rad = sqrtf(xn2) * (1.f + 1e-5f) + max_norm;
        const float eps = kEpsScale * rad * rad;
        const bool unique = (m2 - m1) > eps;
        if (kq == 0 && valid && unique) out_rows[(size_t)n * a.S] = (uint8_t)k1;

        // exact re-score of the ambiguous sub-vectors of this tile
        uint64_t amb = __ballot(kq == 0 && valid && !unique);
        while (amb) {
            const int src = __builtin_ctzll(amb);
            amb &= amb - 1;
            const int64_t nn = n0 + src;
            float xe[G];
            load_subvector<G, CG>(a, nn, h, j, xe);
            float best = INFINITY;
            int bk = 256;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int k = lane + 64 * r;
                const float dist = exact_distance<G, CG>(a, cb, h, j, k, xe);
                if (dist < best) {
                    best = dist;
                    bk = k;
                }
            }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) {
                const float ob = __shfl_xor(best, off);
                const int ok = __shfl_xor(bk, off);
                if (ob < best || (ob == best && ok < bk)) {
                    best = ob;
                    bk = ok;
                }
            }
            if (lane == 0) out_rows[(size_t)nn * a.S] = (uint8_t)bk;
        }
    }
}

template <int G, int CG>
hipError_t launch_gc(const EncodeArgs &a, hipStream_t st) {
    const dim3 grid((unsigned)((a.n_tokens + kTokChunk - 1) / kTokChunk), (a.S + 3) / 4, a.H);
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

bool encode_supported(int G, int cg, int cb_bf16) {
    if (G != 8 && G != 16 && G != 32) return false;
    if (cg != 2 && cg != 4 && cg != 8) return false;
    if (cg > G) return false;
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
