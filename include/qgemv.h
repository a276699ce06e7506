/*
 * qgemv.h -- C ABI of the block-quantized GEMV library for AMD Instinct MI355X
 * (gfx950 / CDNA4).
 *
 * The operation: the decode-step matrix-vector product y = W x over weights
 * stored in a block-scaled quantized format, with the dequantization fused
 * into the weight load.  The source pages build their decode on exactly this
 * (LumenLLM README, feature list: GEMVs for decode and native NVFP4/FP8
 * kernels; bw24 README, feature list: the NVFP4 (W4) decode path with a
 * split-plane repack, a dp4a matvec and per-shape dispatch; memra README,
 * feature list: NVFP4 / Q4_0 / Q8_0 split-plane matvecs).  Formats:
 *
 *   NVFP4  16-element blocks; E2M1 codes (OCP MX v1.0), one E4M3 scale per
 *          block (OCP OFP8 v1.0, the variant without infinities), one fp32
 *          scale per tensor.  w = e2m1(c) * e4m3(s_b) * s_t.
 *   Q8_0   32-element blocks; int8 codes, one fp16 scale.  w = d * q.
 *   Q4_0   32-element blocks; 4-bit codes, one fp16 scale.  w = d * (q - 8).
 *   FP8    E4M3 codes (OCP OFP8 v1.0, the variant without infinities), one
 *          byte per weight, with fp32 scales: one per tensor (QG_FP8_TENSOR)
 *          or one per 128 x 128 tile of W (QG_FP8_B128, the "block-128" FP8
 *          checkpoints of the memra README, loaders entry).  w = e4m3(c) * s.
 *   Q4_K, Q5_K, Q6_K, IQ4_XS  (the K-quant and IQ4_XS formats the pages run
 *          their GGUF models in: memra README, feature list "Decode kernels"
 *          and model table; bw24 README, requirements.  The pages do not
 *          define them; these are the public GGUF definitions, on logical
 *          values.)  256-element super-blocks with an fp16 scale d:
 *          Q4_K / Q5_K  fp16 dmin per super-block, 6-bit scale sc_j and 6-bit
 *                 min m_j per 32 elements, 4- / 5-bit codes q:
 *                 w = d * sc_j * q - dmin * m_j.
 *          Q6_K   int8 scale sc_j per 16 elements, 6-bit codes q:
 *                 w = d * sc_j * (q - 32).
 *          IQ4_XS 6-bit scale ls_j per 32 elements, 4-bit indices q into the
 *                 IQ4_NL codebook T = {-127, -104, -83, -65, -49, -35, -22,
 *                 -10, 1, 13, 25, 38, 53, 69, 89, 113}:
 *                 w = d * (ls_j - 32) * T[q].
 *          k must be a multiple of 256 for these formats.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Logical weight layout is row-major W[n][k]; row r produces output r.
 *    Activations are token-major x[m][k]; outputs y[m][n].
 *  - Ownership: the caller allocates and frees every buffer.  The library
 *    allocates nothing and keeps no state between calls (besides an immutable
 *    device-property cache), so calls are thread-safe and stream-ordered.
 *    The one exception is moe_forward_noalloc, whose workspace is a
 *    library-owned device array per GPU (see there).
 *  - Pointers named "device" must point to device memory of the current HIP
 *    device; "host" pointers to host memory.  Device pointers must be 16-byte
 *    aligned, packed weight buffers 256-byte aligned.  Inputs never alias
 *    outputs.
 *  - stream: a hipStream_t passed as void* (NULL = the default stream).  Every
 *    device entry point only enqueues work: no host synchronisation and no
 *    allocation, so calls may be captured into a HIP graph.
 *  - Errors: every argument check runs on the host before any HIP call; a
 *    failed check returns a negative QG_E* status and enqueues nothing.  A
 *    launch failure returns QG_EHIP (qg_last_hip_error() holds the hipError_t
 *    of the most recent failure).  Faults inside a kernel surface at the
 *    caller's next synchronisation, as for any HIP kernel.
 *  - k must be a positive multiple of 32 for every format (NVFP4's 16-element
 *    blocks come in pairs per 16-byte load); n >= 1.
 *  - Reductions run in a fixed order that depends on k only, never on m, the
 *    grid or timing: results are bitwise reproducible, and token t of a
 *    batch-m call equals, bitwise, a batch-1 call on token t.
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status */
#define QG_OK            0
#define QG_EINVAL       (-1) /* null pointer, bad shape, misalignment, bad code */
#define QG_EUNSUPPORTED (-2) /* shape outside what the kernels implement */
#define QG_EVERSION     (-3) /* packed buffer or descriptor of another layout version */
#define QG_ENOSPC       (-4) /* destination or workspace buffer too small */
#define QG_EHIP         (-5) /* HIP runtime or launch error */

/* ---------------------------------------------------------------- formats */
#define QG_NVFP4 1
#define QG_Q8_0  2
#define QG_Q4_0  3
#define QG_FP8_TENSOR 4
#define QG_FP8_B128   5
#define QG_Q4_K   6
#define QG_Q5_K   7
#define QG_Q6_K   8
#define QG_IQ4_XS 9
#define QG_NVFP4_GATE_UP 10 /* qg_packed_check only: a matrix from qg_pack_nvfp4_gate_up */

#define QG_ABI_VERSION    2
#define QG_LAYOUT_VERSION 2  /* packed device layout described below */
#define QG_MAX_M          16 /* largest token count of the GEMV entry points */

/* ABI and packed-layout versions this library implements. */
int qg_abi_version(void);
int qg_layout_version(void);
/* Static English text for a status code (never NULL). */
const char* qg_status_string(int status);
/* hipError_t of the most recent QG_EHIP return on any thread (0 if none). */
int qg_last_hip_error(void);

/* ------------------------------------------------------ packed layout V2
 * The "split-plane repack" of the pages (bw24 README and memra README, feature
 * lists): codes and scales live in separate planes so that each lane streams
 * 16 contiguous code bytes per load and the scales follow in a plane of their
 * own.  A packed matrix is one buffer:
 *
 *   [codes plane][pad to 256 B][scale plane][pad to 256 B][stamp, 256 B]
 *
 *   The stamp names the layout (the pages' container rejects files of a newer
 *   format version rather than misread them: Lumen landing page, "06 Format"):
 *   uint32 magic 0x4B504751 (the bytes "QGPK"), uint32 layout version
 *   (QG_LAYOUT_VERSION), uint32 format code, uint32 row order (0 logical, 1
 *   gate/up interleaved), int64 n, int64 k; the rest of the 256 bytes zero.
 *   The unpackers and qg_packed_check verify it on the host (QG_EVERSION for
 *   another layout version, QG_EINVAL for a missing stamp or another format,
 *   row order or shape).  The device entry points cannot read device memory
 *   from the host without a synchronisation, so they take a packed device
 *   buffer as this version's layout: a buffer that crosses a version
 *   boundary (a file, another process) is checked with qg_packed_check
 *   before it is uploaded.  The kernels never read the stamp.
 *
 *   NVFP4  codes: n rows of k/2 bytes; byte j of a row holds element 2j in its
 *          low nibble and element 2j+1 in its high nibble.
 *          scales: n rows of k/16 E4M3 bytes, block b covering elements
 *          [16b, 16b+16).
 *   Q4_0   codes: n rows of k/2 bytes; block b occupies bytes [16b, 16b+16)
 *          and byte i of a block holds element 32b+i (low nibble) and element
 *          32b+16+i (high nibble).
 *          scales: n rows of k/32 fp16 bit patterns.
 *   Q8_0   codes: n rows of k int8.  scales: n rows of k/32 fp16 bit patterns.
 *   FP8    codes: n rows of k E4M3 bytes.  scales: fp32; QG_FP8_TENSOR one
 *          value, QG_FP8_B128 a row-major grid [ceil(n/128)][ceil(k/128)]
 *          whose entry (i, j) scales rows [128i, 128i+128) x columns
 *          [128j, 128j+128) (the last tiles may be partial).
 *   K-quants / IQ4_XS, with S = k/256 super-blocks and B = k/32 blocks per row:
 *          codes: n rows of k/2 bytes in the Q4_0 nibble order (the low four
 *          code bits), then for Q5_K k/8 bytes (one dword per block b: bit
 *          8*(e%4) + e/4 holds bit 4 of element 32b+e) or for Q6_K k/4
 *          bytes (two dwords per block: the first for elements e < 16, the
 *          second for e >= 16; with e' = e % 16, bits 8*(e'%4) + 2*(e'/4)
 *          and the next hold bits 4..5 of the code).  Placing four
 *          elements' high bits one byte apart lets the kernel rebuild four
 *          codes with one shift and one mask.
 *          scales: n rows of: the super-block part (Q4_K / Q5_K: S dwords,
 *          d in the low and dmin in the high half; Q6_K / IQ4_XS: S fp16 d),
 *          then the block part (Q4_K / Q5_K: B uint16, sc_b in the low and
 *          m_b in the high byte; Q6_K: the k/16 int8 scales in order;
 *          IQ4_XS: B bytes ls_b).
 * Every row of every plane starts 16-byte aligned when k % 32 == 0.
 */

/* Bytes of a packed matrix (0 if fmt/n/k are invalid). */
size_t qg_packed_bytes(int fmt, int64_t n, int64_t k);

/* Check a packed host buffer (e.g. one read back from a file) against the
 * format and shape the caller expects, before uploading it.  fmt: any format
 * code, or QG_NVFP4_GATE_UP for a fused gate/up matrix of n = 2 * inter rows.
 * QG_OK; QG_EVERSION if the stamp names another layout version; QG_EINVAL for
 * a null buffer, invalid fmt/n/k, a missing stamp, or a stamp of another
 * format, row order or shape; QG_ENOSPC if bytes < qg_packed_bytes. */
int qg_packed_check(int fmt, const void* buf, size_t bytes, int64_t n, int64_t k);
/* Byte offset of the scale plane inside a packed matrix (0 if invalid). */
size_t qg_scale_plane_offset(int fmt, int64_t n, int64_t k);

/* Packers: logical host arrays -> packed host buffer (copy it to the device
 * afterwards).  codes: one code per byte, row-major [n][k] (NVFP4 and Q4_0
 * codes must be 0..15, else QG_EINVAL).  scales: raw bit patterns, row-major
 * [n][k/B].  dst: host, dst_bytes >= qg_packed_bytes(), else QG_ENOSPC.
 * Padding bytes are written as zero.  Exact: unpack(pack(c, s)) == (c, s). */
int qg_pack_nvfp4(const uint8_t* codes, const uint8_t* scales_e4m3, int64_t n, int64_t k,
                  void* dst, size_t dst_bytes);
int qg_pack_q4_0(const uint8_t* codes, const uint16_t* scales_f16, int64_t n, int64_t k,
                 void* dst, size_t dst_bytes);
int qg_pack_q8_0(const int8_t* codes, const uint16_t* scales_f16, int64_t n, int64_t k,
                 void* dst, size_t dst_bytes);

/* Fused gate/up matrix of an MLP for qgemv_nvfp4_swiglu and the MoE experts:
 * logical codes/scales [2*inter][k] with rows [0, inter) the gate projection
 * and rows [inter, 2*inter) the up projection.  The packed matrix has the
 * NVFP4 layout above with the rows interleaved: packed row 2i is gate row i
 * and packed row 2i+1 is up row i, so the two rows that feed output i are one
 * contiguous run of memory.  Same size as qg_packed_bytes(QG_NVFP4, 2*inter, k). */
int qg_pack_nvfp4_gate_up(const uint8_t* codes, const uint8_t* scales_e4m3, int64_t inter, int64_t k,
                          void* dst, size_t dst_bytes);

/* Unpackers: the exact inverse of the packers (host -> host).  Each first
 * verifies the buffer's stamp as qg_packed_check does (QG_EVERSION for a
 * buffer of another layout version). */
int qg_unpack_nvfp4(const void* src, size_t src_bytes, int64_t n, int64_t k,
                    uint8_t* codes, uint8_t* scales_e4m3);
int qg_unpack_nvfp4_gate_up(const void* src, size_t src_bytes, int64_t inter, int64_t k,
                            uint8_t* codes, uint8_t* scales_e4m3);
int qg_unpack_q4_0(const void* src, size_t src_bytes, int64_t n, int64_t k,
                   uint8_t* codes, uint16_t* scales_f16);
int qg_unpack_q8_0(const void* src, size_t src_bytes, int64_t n, int64_t k,
                   int8_t* codes, uint16_t* scales_f16);

/* FP8 packer / unpacker.  fmt: QG_FP8_TENSOR or QG_FP8_B128 (else
 * QG_EINVAL).  codes: E4M3 bit patterns, row-major [n][k]; scales: fp32, 1
 * value (tensor) or the [ceil(n/128)][ceil(k/128)] grid (block-128).  Any
 * bit pattern is accepted (NaN codes decode to NaN).  Exact inverses. */
int qg_pack_fp8(int fmt, const uint8_t* codes, const float* scales, int64_t n, int64_t k,
                void* dst, size_t dst_bytes);
int qg_unpack_fp8(int fmt, const void* src, size_t src_bytes, int64_t n, int64_t k,
                  uint8_t* codes, float* scales);

/* K-quant / IQ4_XS packer and unpacker.  fmt: QG_Q4_K, QG_Q5_K, QG_Q6_K or
 * QG_IQ4_XS; k % 256 == 0.  codes: one per byte, row-major [n][k] (Q4_K and
 * IQ4_XS 0..15, Q5_K 0..31, Q6_K 0..63, else QG_EINVAL).  d: fp16 bits
 * [n][k/256].  dmin: fp16 bits [n][k/256] (Q4_K / Q5_K; ignored otherwise,
 * may be NULL).  sub: Q4_K / Q5_K / IQ4_XS [n][k/32] values 0..63 (else
 * QG_EINVAL), Q6_K [n][k/16] int8 bit patterns.  mins: [n][k/32] 0..63
 * (Q4_K / Q5_K; ignored otherwise, may be NULL).  Exact inverses. */
int qg_pack_kquant(int fmt, const uint8_t* codes, const uint16_t* d, const uint16_t* dmin,
                   const uint8_t* sub, const uint8_t* mins, int64_t n, int64_t k, void* dst,
                   size_t dst_bytes);
int qg_unpack_kquant(int fmt, const void* src, size_t src_bytes, int64_t n, int64_t k, uint8_t* codes,
                     uint16_t* d, uint16_t* dmin, uint8_t* sub, uint8_t* mins);

/* ------------------------------------------------------ dequantization
 * out[r][c] = the weight value, fp32 (device, [n][k]).  NVFP4: e2m1*e4m3 is
 * exact and the product with tensor_scale is rounded once (to nearest even);
 * Q4_0 and Q8_0 values are exact in fp32.  Runs the same device decode code
 * as the GEMV kernels; meant for verification, not for the decode path.
 * tensor_scale is ignored for Q4_0 / Q8_0 / FP8 / K-quants (FP8 values
 * e4m3 * s, and Q4_K / Q5_K values d*sc*q - dmin*m, are rounded once to
 * fp32; Q6_K and IQ4_XS values are exact in fp32). */
int qg_dequant(int fmt, const void* w, float tensor_scale, int64_t n, int64_t k,
               float* out, void* stream);

/* ------------------------------------------------------ fused-dequant GEMVs
 * y[t][r] = sum_c w[r][c] * x[t][c] for t < m, r < n, fp32 accumulation and
 * fp32 output.  1 <= m <= QG_MAX_M (speculative verify of up to K+1 tokens
 * in one batched call, bw24 README, MTP speculative decoding entry; larger m
 * belongs to qgemm_prefill: QG_EUNSUPPORTED).
 *
 * Q8_0 x fp32 activations.  w: device packed Q8_0 [n][k]; x: device fp32
 * [m][k]; y: device fp32 [m][n]. */
int qgemv_q8_0(const void* w, int64_t n, int64_t k, const float* x, int64_t m,
               float* y, void* stream);

/* NVFP4 x bf16 activations.  w: device packed NVFP4 [n][k]; x: device bf16
 * bit patterns [m][k]; y: device fp32 [m][n].  The tensor scale multiplies
 * each row sum. */
int qgemv_nvfp4(const void* w, float tensor_scale, int64_t n, int64_t k,
                const uint16_t* x, int64_t m, float* y, void* stream);

/* FP8 (E4M3) x bf16 activations (LumenLLM README: native FP8 weights; its
 * 9B model runs FP8).  fmt: QG_FP8_TENSOR or QG_FP8_B128; w: device packed
 * FP8 [n][k]; x: device bf16 bit patterns [m][k]; y: device fp32 [m][n].
 * Each 16-element chunk of a row is summed in fp32 (exact products of bf16
 * and e4m3), then added into the row sum as fma(s, chunk_sum, acc) with its
 * tile's scale (block-128), or the row sum is multiplied by the tensor scale
 * once (tensor). */
int qgemv_fp8(int fmt, const void* w, int64_t n, int64_t k, const uint16_t* x, int64_t m, float* y,
              void* stream);

/* NVFP4 fused gate+up GEMV with the SwiGLU epilogue of an MLP.  w_gu: device
 * fused gate/up matrix packed by qg_pack_nvfp4_gate_up (logical rows
 * [0, inter) gate, [inter, 2*inter) up).  a: device bf16 [m][inter] with
 * a = bf16_rne(silu(g) * u), silu(g) = g / (1 + exp(-g)).  h (nullable):
 * device fp32 [m][2*inter] receives g and u (the plain GEMV outputs). */
int qgemv_nvfp4_swiglu(const void* w_gu, float tensor_scale, int64_t inter, int64_t k,
                       const uint16_t* x, int64_t m, uint16_t* a, float* h, void* stream);

/* Q8_0 activation quantizer for the W4A8 path (bw24 README: W4A8 integer
 * path).  Per 32-element block of x (device fp32 [m][k]): amax = max|x|,
 * d32 = amax / 127 (correctly rounded fp32), xd = fp16_rne(d32),
 * xq = clamp(round_half_even(x / d32), -127, 127) (x / d32 correctly
 * rounded), a zero block gives d = 0 and q = 0; xs = sum of xq over the block.
 * xq: device int8 [m][k]; xd: device fp16 bits [m][k/32]; xs (nullable):
 * device int32 [m][k/32].  Any m >= 1. */
int qg_quantize_q8_0_act(const float* x, int64_t m, int64_t k, int8_t* xq, uint16_t* xd,
                         int32_t* xs, void* stream);

/* Q4_0 weights x Q8_0 activations, integer block dots (W4A8).  Per block b:
 * isum_b = sum_j (q_w - 8) * q_x exactly in int32, then
 * y += fp32(d_w) * fp32(d_x) * isum_b in fp32.  w: device packed Q4_0 [n][k];
 * xq/xd/xs as produced by qg_quantize_q8_0_act (xs nullable: then the block
 * sums are recomputed in the kernel); y: device fp32 [m][n]. */
int qgemv_q4_0_a8(const void* w, int64_t n, int64_t k, const int8_t* xq, const uint16_t* xd,
                  const int32_t* xs, int64_t m, float* y, void* stream);

/* W4A8 prefill: Q4_0 weights x Q8_0 activations for any number of tokens
 * on the matrix cores (bw24 README, feature list: the int8 W4A8 tensor-core
 * GEMM for prefill and the int8 expert GEMM).  The same product as
 * qgemv_q4_0_a8 -- per 32-element block the exact int32 dot
 * isum = sum (q_w - 8) * q_x, then acc = fma(d_w * d_x, isum, acc) in fp32,
 * blocks in ascending order -- for m >= 1 (not limited to QG_MAX_M).  Each
 * output depends only on its own token and row: bitwise reproducible and
 * batch-invariant; it agrees with qgemv_q4_0_a8 to rounding (that kernel
 * splits the blocks of a row over lanes).  w: device packed Q4_0 [n][k];
 * xq / xd: device, from qg_quantize_q8_0_act ([m][k] int8, [m][k/32] fp16
 * bits); y: device fp32 [m][n].  m up to 2^24 (else QG_EUNSUPPORTED). */
int qgemm_prefill_a8(const void* w, int64_t n, int64_t k, const int8_t* xq, const uint16_t* xd, int64_t m,
                     float* y, void* stream);

/* K-quant / IQ4_XS weights x Q8_0 activations (memra README, feature list
 * "Decode kernels": K-quant split-plane matvecs with dp4a).  Per 32-element
 * block b of a row, with the block's activation scale d_x, codes q_x and
 * their sum s_x (all from qg_quantize_q8_0_act), exact int32 dots first:
 *   Q4_K / Q5_K  i = sum q * q_x;
 *                y += d_x * fma(d*sc_b, i, -((dmin*m_b) * s_x));
 *   Q6_K         h = sum of q_x over the block's first 16 elements;
 *                v = sc_2b * (sum_lo q*q_x - 32 h)
 *                  + sc_2b+1 * (sum_hi q*q_x - 32 (s_x - h));
 *                y += (d * d_x) * v;
 *   IQ4_XS       v = (ls_b - 32) * sum T[q] * q_x;  y += (d * d_x) * v;
 * blocks in ascending order, then the fixed lane butterfly (fp32).
 * w: device packed [n][k] (k % 256 == 0); xq / xd / xs: device, as written
 * by qg_quantize_q8_0_act (xs is required here); y: device fp32 [m][n]. */
int qgemv_kquant_a8(int fmt, const void* w, int64_t n, int64_t k, const int8_t* xq, const uint16_t* xd,
                    const int32_t* xs, int64_t m, float* y, void* stream);

/* ------------------------------------------------------ MoE decode
 * Router: for each of t tokens pick the top_k largest of n_experts fp32
 * logits (ties to the lower expert index), ordered by logit descending then
 * index ascending; weights = exp(l - l_max) / sum over the selection (the
 * softmax renormalised over the chosen experts).  Selection compares the fp32
 * logits exactly (top-k routing is discontinuous: bw24 README, sigmoid-router
 * MoE entry).  logits: device fp32 [t][n_experts]; ids: device int32
 * [t][top_k]; weights: device fp32 [t][top_k].  1 <= t, 1 <= top_k <= 16,
 * top_k <= n_experts <= 1024.  NaN logits give an unspecified selection. */
int moe_route_topk(const float* logits, int64_t t, int64_t n_experts, int64_t top_k,
                   int32_t* ids, float* weights, void* stream);

#define QG_MOE_KEEP_H 1 /* also store the gate/up outputs h in the workspace */

/* One MoE layer's experts.  Routed experts 0..n_experts-1; when has_shared is
 * 1, expert n_experts is a shared expert that every token uses with weight 1.
 * Every expert has NVFP4 gate_up [2*inter][hidden] (gate rows first) and down
 * [hidden][inter], gate_up packed by qg_pack_nvfp4_gate_up and down by
 * qg_pack_nvfp4; expert e's packed matrices start at gate_up + e *
 * gate_up_stride and down + e * down_stride (device, strides in bytes,
 * multiples of 256, at least qg_packed_bytes of the matrix).  Tensor scales:
 * device fp32 arrays of n_experts + has_shared entries.  layout_version: the
 * packed layout the caller built the experts with; every MoE entry point
 * returns QG_EVERSION before any launch when it is not QG_LAYOUT_VERSION
 * (moe_workspace_bytes and moe_prefill_workspace_bytes return 0). */
typedef struct qg_moe_desc {
    int32_t n_experts;
    int32_t top_k;
    int32_t has_shared;
    int32_t flags;          /* QG_MOE_KEEP_H, or 0 */
    int64_t hidden;
    int64_t inter;
    const void* gate_up;
    int64_t gate_up_stride;
    const void* down;
    int64_t down_stride;
    const float* gate_up_scale;
    const float* down_scale;
    int32_t layout_version; /* QG_LAYOUT_VERSION of the packed experts, else QG_EVERSION */
    int32_t reserved;       /* 0 */
} qg_moe_desc;

/* Workspace bytes moe_gemv_grouped needs for t tokens (0 if d is invalid). */
size_t moe_workspace_bytes(const qg_moe_desc* d, int64_t t);

/* Workspace layout for t tokens, P = t * (top_k + has_shared) pairs (offsets
 * in bytes from ws, each region 256-byte aligned, in this order):
 *   int32 n_groups                 number of active experts incl. shared
 *   int32 experts[P]               active expert ids ascending, shared last
 *   int32 offsets[P + 1]           group g owns pairs [offsets[g], offsets[g+1])
 *   int32 pair_token[P]            token of each pair (ascending within a group)
 *   int32 pair_slot[P]             slot s < top_k, or top_k for the shared expert
 *   uint16 a[P][inter]             bf16 SwiGLU outputs per pair
 *   float h[P][2*inter]            (only with QG_MOE_KEEP_H) gate/up outputs per pair
 *   float o[P][hidden]             down outputs per pair (unweighted)
 *   int32 ids[t][top_k]            (moe_forward) the routing it computed
 *   float weights[t][top_k]        (moe_forward) the routing weights
 * This is the expert-major CSR batching of bw24 README (MoE feature entry):
 * each active expert's weights are streamed once for all its tokens.
 *
 * moe_gemv_grouped: y[t] = sum_s weights[t][s] * down_e(a) + down_shared(a_sh)
 * with a = bf16_rne(silu(g) * u) and [g; u] = gate_up_e(x[t]), expert e =
 * ids[t][s]; the sum runs over slots in ascending order, then the shared
 * expert.  x: device bf16 [t][hidden]; ids/weights: device, as written by
 * moe_route_topk (ids must be distinct per token and < n_experts); y: device
 * fp32 [t][hidden]; ws: device, ws_bytes >= moe_workspace_bytes (else
 * QG_ENOSPC).  1 <= t <= QG_MAX_M, top_k <= 8, hidden and inter multiples of
 * 32.  Routing never returns to the host (the pages' decode keeps its
 * per-token host traffic to a few bytes: bw24 README, CUDA-graph decode). */
int moe_gemv_grouped(const qg_moe_desc* d, const uint16_t* x, const int32_t* ids,
                     const float* weights, int64_t t, float* y, void* ws, size_t ws_bytes,
                     void* stream);

/* The whole MoE layer from router logits in two launches: the gate/up kernel
 * first routes every token itself (exactly as moe_route_topk, so ids and
 * weights are bitwise the same) and writes ids/weights into the workspace,
 * then the grouped GEMVs and the combine run as in moe_gemv_grouped.  The
 * result equals moe_route_topk followed by moe_gemv_grouped, bitwise.
 * logits: device fp32 [t][n_experts] (n_experts <= 1024).  Other arguments as
 * for moe_gemv_grouped. */
int moe_forward(const qg_moe_desc* d, const uint16_t* x, const float* logits, int64_t t, float* y,
                void* ws, size_t ws_bytes, void* stream);

/* moe_forward without a caller workspace.  For callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid hipMalloc.  The workspace lives in a library-owned
 * device array of QG_MOE_NOALLOC_SCRATCH_BYTES per GPU (allocated with the
 * library's code object on each device it runs on, held until the process
 * ends); the call itself allocates nothing.  Same result as moe_forward,
 * bitwise (the same kernels on the same workspace layout).  QG_ENOSPC when
 * moe_workspace_bytes(d, t) exceeds QG_MOE_NOALLOC_SCRATCH_BYTES (the 257-
 * expert, hidden 2048, inter 512 layer needs 1.4 MB at t = 16, 2.0 MB with
 * QG_MOE_KEEP_H).  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (other streams, other threads) race and must be
 * serialised by the caller.  The array keeps the last call's workspace; no
 * region needs clearing between calls.  Other arguments as for moe_forward;
 * QG_EHIP if the array's device address cannot be obtained. */
#define QG_MOE_NOALLOC_SCRATCH_BYTES (4 << 20)
int moe_forward_noalloc(const qg_moe_desc* d, const uint16_t* x, const float* logits, int64_t t, float* y,
                        void* stream);

/* ------------------------------------------------------ MoE prefill
 * The same MoE layer as moe_forward (same routing, grouping, SwiGLU and
 * combine definitions and the same result up to rounding) for many tokens:
 * the grouped NVFP4 MoE GEMM of the LumenLLM README's prefill (feature list
 * "Kernels").  The expert matmuls run on the matrix cores over tiles of up to
 * 32 pairs of one expert: bf16 activations times exactly decoded weights,
 * fp32 accumulation (two partial sums per output added in a fixed order),
 * then the tensor scale; a = bf16_rne(silu(g) * u).  A pair's products do not
 * depend on which tile it lands in, so results are bitwise reproducible and a
 * token's output does not depend on the other tokens of the call.
 * 1 <= t <= 65536, top_k <= 8, n_experts <= 1024; hidden and inter each one
 * of 512, 1024, 2048 (else QG_EUNSUPPORTED).  The workspace starts with the
 * moe_gemv_grouped / moe_forward layout above for these P = t * (top_k +
 * has_shared) pairs (the CSR, a, h with QG_MOE_KEEP_H, o, ids, weights),
 * followed by int32 tile_start[P + 2], int32 counts[n_experts], int32
 * pair_pos[t][top_k + 1] and int32 tiles[T + 1][4] with T = ceil(t * top_k /
 * 32) + min(n_experts, t * top_k) + (has_shared ? ceil(t / 32) : 0): the
 * tile count in tiles[0][0], then per 32-pair GEMM tile its expert, first
 * pair and pair count (each region 256-byte aligned).  Five launches on the
 * stream: routing, pair counting and placement, gate/up + SwiGLU, down,
 * combine. */
size_t moe_prefill_workspace_bytes(const qg_moe_desc* d, int64_t t);
int moe_prefill(const qg_moe_desc* d, const uint16_t* x, const float* logits, int64_t t, float* y,
                void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------ small-M prefill GEMM
 * Y[t][r] = bf16_rne(s_t * sum_c D[r][c] * X[t][c]) with D = e2m1 * e4m3
 * (exact in bf16), bf16 matrix-core products and fp32 accumulation; the
 * prefill counterpart of the decode GEMV over the same packed NVFP4 weights
 * (LumenLLM README, feature list: NVFP4 prefill GEMMs; memra README, known
 * gaps: prefill keeps bf16 activations rather than W4A4 numerics).
 * w: device packed NVFP4 [n][k]; x: device bf16 [m][k]; y: device bf16
 * [m][n].  Any m >= 1.  For m <= 128 with k a multiple of 256 one launch
 * reads every weight byte once (48 weight rows and all tokens a workgroup);
 * there a row's result does not depend on the other rows or on m. */
int qgemm_prefill(const void* w, float tensor_scale, int64_t n, int64_t k, const uint16_t* x,
                  int64_t m, uint16_t* y, void* stream);

/* Device workspace bytes that qgemm_prefill_ws needs for this shape: nonzero
 * for m <= 128 with k not a multiple of 256 (ceil(k / 1024) * m * n fp32
 * partial sums), 0 when the shape runs without one (m > 128, or k a multiple
 * of 256), and 0 for invalid arguments. */
size_t qgemm_prefill_workspace_bytes(int64_t n, int64_t k, int64_t m);

/* The same product as qgemm_prefill, with a caller-owned device workspace.
 * For m <= 128 with k not a multiple of 256 the k range is split into slices
 * of 1024 handled by separate workgroups (each reads only its slice of x, the
 * dominant memory traffic of a small-m product); their fp32 partial sums go
 * to ws and a second launch adds them in slice order and rounds once.  Every
 * other shape runs qgemm_prefill's kernels (bitwise its result) and leaves ws
 * untouched.  ws: device, 256-byte aligned,
 * ws_bytes >= qgemm_prefill_workspace_bytes(n, k, m) (else QG_EINVAL for a
 * null or misaligned ws, QG_ENOSPC for too few bytes); ignored (may be null)
 * when that size is 0.  The library reads and writes ws only during the call
 * (stream-ordered); calls that share a workspace must not overlap.  A row's
 * result does not depend on the other rows or on m within m <= 128; with the
 * split k it agrees with qgemm_prefill to rounding (the summation order
 * differs). */
int qgemm_prefill_ws(const void* w, float tensor_scale, int64_t n, int64_t k, const uint16_t* x,
                     int64_t m, uint16_t* y, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------ kernel policy
 * The one rollback seam (the pages keep configuration flags only for runtime
 * parameters, machine configuration and rollback seams: memra README, quick
 * start, flag catalog).  QG_KERNEL_TUNED, the default, runs the
 * shape-specialised kernels.  QG_KERNEL_GENERIC sends the calls that have
 * one to a simpler kernel of the same family:
 *   qgemv_nvfp4 / qgemv_nvfp4_swiglu at m = 1: the chunk-loop kernel of
 *     m = 2..16 rather than the streaming kernel (bitwise the same result);
 *   moe_gemv_grouped / moe_forward / moe_forward_noalloc at 2..4 tokens: the
 *     per-(expert group, row tile) kernels of one token rather than the
 *     row-tile kernels (bitwise the same result);
 *   qgemm_prefill_ws at m <= 128 with k not a multiple of 256: the kernel
 *     of qgemm_prefill (the workspace is left untouched; the result is
 *     qgemm_prefill's, which agrees with the split-k result to rounding).
 * Every other call is unaffected.  The initial policy comes from the
 * environment variable QG_FORCE_KERNEL ("generic" or "tuned"; anything else,
 * or unset, is tuned), read once, when the library is first used.
 * qg_set_kernel_policy changes it for the whole process from the next call
 * on (work already enqueued keeps its kernels); it returns QG_OK, or
 * QG_EINVAL for an unknown policy.  qg_kernel_policy returns the current
 * one. */
#define QG_KERNEL_TUNED   0
#define QG_KERNEL_GENERIC 1
int qg_set_kernel_policy(int policy);
int qg_kernel_policy(void);

/* ------------------------------------------------------ achievable-peak probes
 * Measurement tools, not part of the decode path: what this GPU reaches with
 * the instructions the kernels use, printed beside the data-sheet peaks (the
 * pages keep such microbenchmarks next to their kernels: bw24 README, crate
 * table, the probe crate; memra README, research notes, microbenched peaks).
 *
 * qg_probe_read: stream `bytes` of the device buffer buf once (16-byte
 * non-temporal loads, eight in flight per lane, 1 KB contiguous per wave-wide
 * load) with wg_per_cu (1..8) four-wave workgroups per compute unit; time it
 * on the stream for the achievable HBM read bandwidth.  buf: device, 16-byte
 * aligned, bytes a positive multiple of 16; sink: device uint32, written only
 * in the (practically impossible) case that the folded data equals a fixed
 * key, so that the loads are not optimised away.
 *
 * qg_probe_mfma_bf16: iters rounds of sixteen independent
 * v_mfma_f32_16x16x32_bf16 per wave, eight waves per compute unit, no memory
 * traffic; *flops (host) receives the floating-point operations launched
 * (2 * 16 * 16 * 32 per MFMA).  sink: device float, written only if the
 * result equals a fixed key.  1 <= iters <= 2^32. */
int qg_probe_read(const void* buf, size_t bytes, int wg_per_cu, uint32_t* sink, void* stream);
int qg_probe_mfma_bf16(int64_t iters, float* sink, int64_t* flops, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
