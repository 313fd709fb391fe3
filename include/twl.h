/*
 * twl.h -- C ABI of the MI355X (gfx950) ternary linear layer library.
 *
 * The operation (pages cited by title and section):
 *   [P1] "Ternary-Bonsai-2-27B on 2x RTX 5070 with vLLM TP=2"
 *        (qiita.com/nakanokensetsu/items/ecc183fae033565af7cb)
 *        Prerequisites -- weights are {-1,0,+1} in 2 bits with one scale per
 *          128 elements; a block-wise Hadamard rotation sits on the input side.
 *        Section 1 -- the rotation's sign table is keyed by the full input
 *          width; H1024 [a; b] = [H512 a + H512 b ; H512 a - H512 b].
 *        Section 4 (prefill linear layers to an int8 GEMM) -- s[n,g] is split
 *          as q[n,g] = round(127 s[n,g] / smax[n]); W_int8 = code * q fits int8;
 *          the matmul becomes one int8 GEMM with int32 accumulation plus a
 *          per-row and per-token rescale; activations are quantised to int8
 *          per token after the rotation.
 *        Section 5 (what did not help) -- a dp4a decode GEMV.
 *
 * Conventions shared by every entry point
 *   - All array arguments are DEVICE pointers on the current HIP device, owned
 *     by the caller, contiguous and row-major, at least 16-byte aligned.  The
 *     library allocates nothing and keeps no per-call state.
 *   - Work is enqueued on `stream` (NULL = the legacy default stream) and is
 *     asynchronous; nothing synchronises.  Outputs are valid once the stream
 *     reaches that point.
 *   - Shape, null-pointer and alignment errors are detected on the host before
 *     anything is enqueued and return a non-zero status; twl_last_error() then
 *     holds a message (thread-local).  A failed launch returns TWL_EHIP.
 *     Faults inside kernels surface at the caller's next synchronisation.
 *   - K must be a positive multiple of 1024 (whole Hadamard blocks) and at
 *     most TWL_MAX_K; M and N may be any value >= 0 (0 enqueues nothing).
 *   - Non-finite activations or scales give unspecified results.
 */
#ifndef TWL_H
#define TWL_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TWL_OK = 0,
  TWL_EINVAL = 1,   /* null pointer, negative size, bad enum value        */
  TWL_ESHAPE = 2,   /* K not a multiple of 1024, K > TWL_MAX_K, too large  */
  TWL_EALIGN = 3,   /* a pointer is not 16-byte aligned                    */
  TWL_EDEVICE = 4,  /* the current device is not gfx950                   */
  TWL_EHIP = 5      /* a HIP runtime call or kernel launch failed          */
} twl_status;

#define TWL_HBLOCK 1024      /* Hadamard block width along K              */
#define TWL_GROUP 128        /* K elements per weight scale group         */
#define TWL_MAX_K 65536      /* 64 blocks; |acc| <= 127*127*K < 2^31       */
#define TWL_GEMV_MAX_M 24    /* decode batches up to this size use a decode kernel */

/* Which kernel family computes the linear layer (twl_ternary_linear_ex). */
typedef enum {
  TWL_PATH_AUTO = 0,       /* decode kernel for M <= TWL_GEMV_MAX_M, else the GEMM */
  TWL_PATH_GEMM = 1,       /* int8-MFMA GEMM with in-register 2-bit unpack         */
  TWL_PATH_GEMV = 2,       /* decode kernel (M <= TWL_GEMV_MAX_M), chosen by shape */
  TWL_PATH_GEMV_DOT4 = 3,  /* decode: packed-2-bit dot4 GEMV, no matrix cores      */
  TWL_PATH_GEMV_MFMA = 4   /* decode: int8 MFMA over the stream (tokens padded to 16 or 32) */
} twl_path;

/*
 * rotate_quant_act -- [P1] Prerequisites, section 1 and section 4.
 *   For every token t and 1024-block b:
 *     r[t, 1024b:1024b+1024] = (1/32) * H1024 * (sign[1024b:...] * x[t, ...])
 *   with H1024 the Sylvester Hadamard matrix, evaluated as an fp32 fast
 *   Walsh-Hadamard transform with stages h = 1, 2, ..., 512 (each butterfly
 *   (lo, hi) -> (lo + hi, lo - hi)).  Then, per token over the whole row:
 *     a_scale[t] = max_k |r[t,k]| / 127              (fp32, IEEE division)
 *     x_i8[t,k]  = clamp(rint(r[t,k] / a_scale[t]), -127, 127)  (ties to even)
 *   An all-zero token gives a_scale = 0 and x_i8 = 0.
 *   x       in : bf16 bit patterns [M, K]
 *   sign    in : int8 [K], each +1 or -1 (one table per input width)
 *   x_i8    out: int8 [M, K]
 *   a_scale out: fp32 [M]
 */
twl_status twl_rotate_quant_act(const uint16_t* x, const int8_t* sign, int64_t M, int64_t K,
                                int8_t* x_i8, float* a_scale, hipStream_t stream);

/*
 * silu_mul_rotate_quant_act -- the down projection's input step, fused:
 * rotate_quant_act applied to act = bf16(SiLU(gate) * up), where gate and up
 * are the two halves of the gate/up projection's output.  [P1] section 1 names
 * the model's 17408-wide intermediate layer; its gated SiLU activation is this
 * library's reading, as is the exact evaluation:
 *   e = exp(-g) by a fixed fp32 sequence (argument clamped to [-87, 88],
 *       n = rint(x log2 e), r = (x - n * 0x1.62e4p-1) - n * 0x1.7f7d1cp-20,
 *       Taylor polynomial of degree 7 in Horner form, times 2^n),
 *   s = g / (1 + e) (IEEE division), act = bf16(s * up) (nearest even),
 * every step in fp32 without fused multiply-adds, so the result is bit-exact
 * to an unfused pipeline that evaluates the same steps.
 *   gate_up in : bf16 bit patterns [M, 2K]; gate = columns 0..K-1, up = K..2K-1
 *   sign    in : int8 [K]
 *   x_i8    out: int8 [M, K];  a_scale out: fp32 [M]   (as rotate_quant_act)
 * Same errors as rotate_quant_act (K % 1024, K <= TWL_MAX_K, alignment).
 */
twl_status twl_silu_mul_rotate_quant_act(const uint16_t* gate_up, const int8_t* sign, int64_t M,
                                         int64_t K, int8_t* x_i8, float* a_scale,
                                         hipStream_t stream);

/*
 * pack_ternary -- [P1] Prerequisites and section 4 (load time, once per weight).
 *   smax[n]  = max_g |s[n,g]|                               (fp32, exact)
 *   q[n,g]   = rint((127 * s[n,g]) / smax[n])  in fp32, ties to even; 0 if smax = 0
 *   packed   : 2 bits per code, field u = 0 for -1, 1 for +1, 2 for 0 (four
 *              codes per byte).  A row's codes form K/16 little-endian 32-bit
 *              words, code k = 16w + 4i + b in bits [8b + 2i, 8b + 2i + 1] of
 *              word w.  The 8 words (32 bytes) of row n and group g = k/128
 *              are stored at byte ((n/64) * K/128 + g) * 2048 + (n%64) * 32:
 *              2 KB tiles of 64 rows x one group, ceil(N/64) row blocks, rows
 *              past N padded with code 0 (bytes 0xAA).  This layout is the
 *              library's own (the pages fix only 2 bits per code).
 *   code      in : int8 [N, K], values in {-1, 0, +1}
 *   s         in : fp16 bit patterns [N, K/128]
 *   packed    out: uint8, twl_packed_bytes(N, K) bytes
 *   q         out: int8 [N, K/128], |q| <= 127
 *   smax      out: fp32 [N]
 *   bad_codes out: optional (may be NULL) device int32 counter; the number of
 *              codes outside {-1,0,+1} is ADDED to it.  Such codes pack as 0.
 */
twl_status twl_pack_ternary(const int8_t* code, const uint16_t* s, int64_t N, int64_t K,
                            uint8_t* packed, int8_t* q, float* smax, int32_t* bad_codes,
                            hipStream_t stream);

/*
 * Size in bytes of the packed weight buffer of an N x K layer:
 * ceil(N/64) * 64 * K/4 (0 for N <= 0 or an invalid K).
 */
size_t twl_packed_bytes(int64_t N, int64_t K);

/*
 * Bytes of workspace twl_ternary_linear* may need for this shape on the
 * current device (0 = none; valid for every path).  The workspace holds int32
 * partial sums: the GEMM's split-K tiles, or the decode GEMV's per-slice sums
 * when it splits K across workgroups.  Its contents on entry do not matter
 * (no clearing needed); calls sharing a workspace must not run concurrently.
 */
size_t twl_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * ternary_linear -- [P1] section 4 (prefill GEMM) and section 5 (decode).
 *   acc[t,n] = sum_k x_i8[t,k] * code[n,k] * q[n, k/128]      (exact int32)
 *   y[t,n]   = acc[t,n] * a_scale[t] * smax[n] / 127           (fp32)
 *   Prefill sizes run an int8-MFMA GEMM that unpacks the 2-bit codes on chip;
 *   decode batches (M <= TWL_GEMV_MAX_M) stream the packed weights through an
 *   int8 MFMA kernel, tokens padded to 16 (M <= 16) or 32 (every CU an equal
 *   range of rows when each CU gets at least 16 rows) or, for narrower
 *   layers, a dot4 GEMV
 *   (M < 4) or a K-split MFMA kernel.  All give
 *   bit-identical acc.
 *   x_i8 [M,K], a_scale [M], packed (twl_packed_bytes(N,K) bytes), q [N,K/128],
 *   smax [N] as produced by the two calls above; y out: fp32 [M, N].
 *   workspace: device memory of at least twl_workspace_bytes(M,N,K) bytes; may
 *   be NULL when that is 0.
 */
twl_status twl_ternary_linear(const int8_t* x_i8, const float* a_scale, const uint8_t* packed,
                              const int8_t* q, const float* smax, int64_t M, int64_t N, int64_t K,
                              float* y, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * ternary_linear_acc -- the same kernels with the rescale left out: writes the
 * exact int32 accumulators acc [M, N] (for bit-exact verification).
 */
twl_status twl_ternary_linear_acc(const int8_t* x_i8, const uint8_t* packed, const int8_t* q,
                                  int64_t M, int64_t N, int64_t K, int32_t* acc,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * rotate_act_bf16 -- the rotation of rotate_quant_act alone (same sign and
 * block FWHT, same fp32 operations), without the int8 step: r rounded to bf16
 * (nearest even).  The input of the bf16 reference linear below.
 *   x in: bf16 bit patterns [M, K];  sign in: int8 [K];  r out: bf16 bits [M, K]
 */
twl_status twl_rotate_act_bf16(const uint16_t* x, const int8_t* sign, int64_t M, int64_t K,
                               uint16_t* r, hipStream_t stream);

/*
 * reference_linear_bf16 -- [P1] section 4, the bf16 path the int8 GEMM
 * replaced (kept as an accuracy reference and an A/B point):
 *   y[t,n] = sum_k r[t,k] * code[n,k] * bf16(s[n, k/128])    (fp32 accumulation)
 * with the weights expanded from the packed codes and the ORIGINAL fp16 scales
 * in registers (s rounded to bf16, nearest even).  Not the hot path: no
 * workspace, no split-K, one untuned kernel.
 *   r      in : bf16 bit patterns [M, K] (from twl_rotate_act_bf16)
 *   packed in : twl_packed_bytes(N, K) bytes (from twl_pack_ternary)
 *   s      in : fp16 bit patterns [N, K/128]
 *   y      out: fp32 [M, N]
 */
twl_status twl_reference_linear_bf16(const uint16_t* r, const uint8_t* packed, const uint16_t* s,
                                     int64_t M, int64_t N, int64_t K, float* y,
                                     hipStream_t stream);

/* What twl_ternary_linear_ex writes into `out` [M, N]. */
typedef enum {
  TWL_OUT_F32 = 0,      /* y, fp32                                              */
  TWL_OUT_ACC_I32 = 1,  /* the exact int32 accumulators (no rescale)            */
  TWL_OUT_BF16 = 2      /* y rounded to bf16 (nearest even), as uint16 bit patterns;
                           the same fp32 value as TWL_OUT_F32 before rounding   */
} twl_out;

/*
 * ternary_linear_ex -- explicit output kind and kernel family.  out_kind is a
 * twl_out: with TWL_OUT_ACC_I32, a_scale and smax are ignored and may be NULL.
 * The bf16 output halves the bytes of y, which dominate the prefill step's
 * traffic (the pages' consumers take bf16 activations, [P1] section 4).
 * The decode paths (TWL_PATH_GEMV, _GEMV_DOT4, _GEMV_MFMA) require
 * M <= TWL_GEMV_MAX_M; TWL_PATH_GEMV picks the row-balanced MFMA kernel
 * when each CU gets at least 16 rows, else the dot4 kernel for M < 4 and the
 * K-split MFMA kernel above.  TWL_PATH_GEMV_MFMA forces a matrix-core decode
 * kernel (row-balanced when it applies) and TWL_PATH_GEMV_DOT4 the dot4
 * kernel.  All paths give bit-identical acc.
 */
twl_status twl_ternary_linear_ex(const int8_t* x_i8, const float* a_scale, const uint8_t* packed,
                                 const int8_t* q, const float* smax, int64_t M, int64_t N, int64_t K,
                                 void* out, int out_kind, int path,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * ternary_linear_noalloc -- for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same computation, kernels and results as
 * twl_ternary_linear_ex (same arguments, same errors) without the workspace
 * argument: K-split partial sums go to a scratch buffer the library owns, a
 * static device array of TWL_NOALLOC_SCRATCH_BYTES on each GPU the library
 * runs on (held until the process ends).  No call allocates or frees
 * anything.  A shape whose plan needs more scratch than that returns
 * TWL_ESHAPE (twl_workspace_bytes gives the need; use twl_ternary_linear_ex
 * with a workspace for such shapes).  Every call on one GPU shares its
 * scratch: calls that may overlap on one GPU (different streams, or
 * different host threads) race and must be serialised by the caller.  The
 * scratch needs no clearing: each call writes every partial sum it reads.
 */
#define TWL_NOALLOC_SCRATCH_BYTES (32u << 20)
twl_status twl_ternary_linear_noalloc(const int8_t* x_i8, const float* a_scale,
                                      const uint8_t* packed, const int8_t* q, const float* smax,
                                      int64_t M, int64_t N, int64_t K, void* out, int out_kind,
                                      int path, hipStream_t stream);

/*
 * plan_info -- the kernels twl_ternary_linear_ex would launch for this shape
 * and path on the current device, without launching anything (for tests and
 * tuning; the choice is a function of M, N, K, path and the CU count only).
 * Writes eight values to info (host memory, caller-owned):
 *   info[0] kernel family: 1 = prefill GEMM, 2 = row-balanced MFMA decode,
 *           3 = dot4 decode, 4 = K-split MFMA decode
 *   info[1] GEMM block-tile rows, or (decode) rows per workgroup at most
 *   info[2] GEMM block-tile columns (0 for decode)
 *   info[3] K splits: GEMM split-K count or decode K slices (1 = not split)
 *   info[4] workgroups of the main kernel
 *   info[5] waves per workgroup
 *   info[6] 1 when a second (reduce) kernel follows, else 0
 *   info[7] workspace bytes this path needs
 * M = 0 or N = 0 writes zeros.  Errors as twl_ternary_linear_ex (shape, path,
 * decode batch limit), TWL_EINVAL for a NULL info, TWL_EDEVICE / TWL_EHIP
 * when the current device is not a usable gfx950.
 *
 * Diagnostics: with the environment variable TWL_LOG set, every linear call
 * (ternary_linear and its variants, rotate_quant_linear) also prints its plan
 * on stderr, one line beginning "[twl]" (for the
 * decode row kernel including its subtile form, token operands, groups of
 * loads in flight per wave and early issue).  The format is for people and
 * tests, not a stable interface.
 */
twl_status twl_plan_info(int64_t M, int64_t N, int64_t K, int path, int64_t* info);

/*
 * rotate_quant_linear -- a whole ternary linear layer from its bf16 input:
 * rotate_quant_act ([P1] Prerequisites, sections 1 and 4; with silu = 1
 * silu_mul_rotate_quant_act, x then being the gate/up output [M, 2K]) followed
 * by ternary_linear_ex with TWL_PATH_AUTO ([P1] section 4 for prefill, section
 * 5 for decode).  x_i8, a_scale and out are all written and are bit-identical
 * to what the two calls produce.
 *   x         in : bf16 bit patterns [M, K] (silu = 1: [M, 2K])
 *   sign      in : int8 +-1 [K]
 *   packed, q, smax in: as ternary_linear
 *   x_i8      out: int8 [M, K];  a_scale out: fp32 [M]  (device, caller-owned)
 *   out       out: [M, N] of the out_kind (twl_out)
 *   workspace     : as ternary_linear_ex for this M, N, K (twl_workspace_bytes)
 * For small decode batches (at most 2 tokens, K <= 17408, at most 2 1024-blocks
 * of rotation per wave of a decode workgroup, 3 for a single token, on shapes
 * where the row-balanced decode kernel covers N with one workgroup per CU)
 * one fused kernel does both steps: every decode
 * workgroup rotates and quantises the tokens itself while its first weight
 * loads are in flight, which removes the rotation's own launch from the
 * decode step.  Other shapes run the two kernels back to back on `stream`.
 * twl_rotate_quant_linear_fused tells which applies.  Errors: those of both
 * steps, checked before anything is enqueued; TWL_EINVAL for silu not 0 or 1.
 * M = 0 is a no-op; N = 0 writes only x_i8 and a_scale.
 */
twl_status twl_rotate_quant_linear(const uint16_t* x, const int8_t* sign, const uint8_t* packed,
                                   const int8_t* q, const float* smax, int64_t M, int64_t N,
                                   int64_t K, int silu, int8_t* x_i8, float* a_scale, void* out,
                                   int out_kind, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/*
 * rotate_quant_linear_fused -- 1 when twl_rotate_quant_linear runs this shape
 * as one fused kernel on the current device, 0 when it runs the two steps, or
 * a negative twl_status (-TWL_ESHAPE, -TWL_EDEVICE, ...) for a shape or device
 * it rejects.
 */
int twl_rotate_quant_linear_fused(int64_t M, int64_t N, int64_t K);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* twl_last_error(void);

/* ABI version of this header (bumped on incompatible changes). */
int twl_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TWL_H */
