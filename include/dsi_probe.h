/*
 * dsi_probe.h — the device converters the indexer kernels rely on, run over
 * their whole input ranges so that tests can compare them with the CPU
 * oracle.
 *
 * Not part of the indexer path: a separate library (libdsi_probe.so) that
 * only the tests load.  Each probe calls the same inline device functions the
 * kernels call (sparse_attention_token_amd/csrc/common.h):
 *   - fp32 -> OCP E4M3FN on v_cvt_pk_fp8_f32 (the q quantization of P3 step
 *     ④, "DeepSeek V3.2 稀疏注意力 DSA 推理流程图解");
 *   - E4M3FN -> f16 (every logits kernel's operand decode) and -> bf16 (the
 *     MXFP4 kernels' q decode);
 *   - FP4 E2M1 x E8M0 block scale -> bf16 (the MXFP4 key decode of P1 "V4.1
 *     索引器接入稀疏 MQA logits").
 * Conventions: device pointers owned by the caller; each call enqueues one
 * kernel on `stream` and returns 0, or a negative dsi status (dsi.h) for
 * rejected arguments (nothing is enqueued then).
 */
#ifndef DSI_PROBE_H
#define DSI_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSI_PROBE_API __attribute__((visibility("default")))

/*
 * The E4M3FN code of every fp32 bit pattern u0 + i, i < n (no wrap past
 * 2^32), on the hardware encoder, reported as its changes: first[0] = the
 * code of u0; every i > 0 whose code differs from that of i - 1 adds the pair
 * (u0 + i, code) to `trans` (uint32 [cap][2], in no particular order) and
 * counts in *ntrans (which the caller zeroes; counts past cap are not
 * stored).  Between two reported changes the code is constant.
 * Errors: DSI_EINVAL (nulls, n < 1, u0 + n > 2^32).
 */
DSI_PROBE_API int dsip_e4m3_encode_changes(uint32_t u0, int64_t n, uint32_t* trans, uint32_t cap, uint32_t* ntrans,
                                           uint32_t* first, hipStream_t stream);

/* f16 bits (uint16 [256]) and bf16 bits (uint16 [256]) of every E4M3FN code. */
DSI_PROBE_API int dsip_e4m3_decode_all(uint16_t* f16_out, uint16_t* bf16_out, hipStream_t stream);

/*
 * bf16 bits of every FP4 E2M1 code times every E8M0 scale: out uint16
 * [256][16], row E (scale 2^(E-127), E = 0 the subnormal 2^-127), column =
 * the code.
 */
DSI_PROBE_API int dsip_fp4_decode_all(uint16_t* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSI_PROBE_H */
