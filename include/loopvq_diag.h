/*
 * libloopvq diagnostics: entry points that expose an intermediate quantity
 * of a kernel so that its numerical error can be measured.  Same conventions
 * as loopvq.h (C ABI, caller-owned device buffers, asynchronous on `stream`).
 */
#ifndef LOOPVQ_DIAG_H
#define LOOPVQ_DIAG_H

#include "loopvq.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * lvq_encode, and also every screen value the encoder's MFMA screen forms
 * (the nearest-codeword search of the LoopVQ project page, "Component 1 --
 * Loop-axis vector quantization"; the news article "How LoopVQ works").  The
 * screen value of code k for sub-vector x is |c_k|^2 - 2 x . c_k: the squared
 * distance minus |x|^2, the same for every code, contracted on the matrix
 * cores in fp32.  The encoder trusts its screen winner when the two smallest
 * screen values are further apart than a bound on the screen's error; these
 * values let that error be measured against an exact evaluation.
 *
 * The run is always encoded through the screen (also runs of at most 32
 * tokens, which lvq_encode evaluates directly); the indices written are those
 * of lvq_encode.  screen: device fp32 [n_tokens][Hk][S][256], 16-byte
 * aligned; entry (n, h, j, k) is the screen value of code k for sub-vector j
 * of token n and KV head h, before the encoder's bookkeeping touches it.
 * Models with n_loops > loop_steps: LVQ_ERR_UNSUPPORTED.  Other arguments and
 * errors as for lvq_encode (LVQ_ERR_INVALID_ARG also for a null or
 * misaligned screen).
 */
lvq_status lvq_encode_screen(const lvq_config *cfg, const void *x, const int64_t *x_strides,
                             int64_t n_tokens, const void *codebook, uint8_t *index_cache,
                             int32_t seq, int64_t first_token, float *screen, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LOOPVQ_DIAG_H */
