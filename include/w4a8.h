/*
 * w4a8.h — C ABI of the MI355X (gfx950) W4A8 linear layer.
 *
 * The operation is the W4A8 GEMM of QServe/QoQ (page "[Feature] Support
 * W4A8KV4 Quantization(QServe/QoQ)", quoted abstract): 4-bit weights reached
 * by a progressive (two-level) quantization, 8-bit per-token activations, an
 * 8-bit integer matrix product, and no dequantization of partial sums.
 * The pages give no formula; this library implements the reading below.
 *
 *   level 1 (per output row n):  s1[n] = fp16(absmax_k |W[n,k]| / 119),
 *                                W8 = clamp(rint(W * fp32(1/s1)), -119, 119)
 *   level 2 (per group of g k):  s2 = max(1, ceil((hi-lo)/15)) in [1,16],
 *                                z = rne(-lo/s2) in [0,15], with lo/hi the
 *                                group's min/max widened to include 0,
 *                                q = clamp(rne(W8/s2) + z, 0, 15)
 *   decode (in the GEMM):        W8^ = (q - z) * s2, always inside int8
 *   per-channel mode (g = K):    s1[n] = fp16((hi-lo)/15) over the row, q and z
 *                                per row, s2 = 1
 *   activations (per token m):   s_a[m] = fp16(absmax_k |A[m,k]| / 127),
 *                                A8 = clamp(rint(A * fp32(1/s_a)), -127, 127)
 *   GEMM:                        acc[m,n] = sum_k A8[m,k] * W8^[n,k]  (int32, exact)
 *                                Y[m,n]   = fp16(acc * s_a[m] * s1[n])  (fp32 math)
 *
 * Conventions for every entry point
 *   - All matrices are row-major.  W is N x K (output x input, as a linear
 *     layer stores it), A is M x K, Y is M x N.
 *   - fp16 values are passed as raw IEEE binary16 bit patterns (uint16_t).
 *   - Pointers named *_dev are device (HBM) pointers; all others are host.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     GPU entry points only enqueue work: they do not synchronize, allocate,
 *     free, or keep state between calls.  The caller owns every buffer.
 *   - Arguments are validated on the host before any HIP call.  A rejected
 *     call returns an error status and touches no memory.  A failed kernel
 *     launch returns W4A8_ERR_DEVICE; faults inside a kernel surface at the
 *     caller's next synchronization, as usual for HIP.
 *   - No entry point throws.
 */
#ifndef W4A8_H
#define W4A8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  W4A8_OK = 0,
  W4A8_ERR_INVALID_ARGUMENT = 1,   /* null pointer, negative size, ld too small, misaligned */
  W4A8_ERR_UNSUPPORTED = 2,        /* shape or group size outside what the kernels handle */
  W4A8_ERR_BUFFER_TOO_SMALL = 3,   /* blob or workspace smaller than required */
  W4A8_ERR_NONFINITE = 4,          /* w4a8_pack: a weight is NaN or infinite */
  W4A8_ERR_RANGE = 5,              /* w4a8_pack: a scale overflows fp16 */
  W4A8_ERR_LAYOUT = 6,             /* blob header magic/version/shape mismatch */
  W4A8_ERR_DEVICE = 7              /* a HIP call failed */
} w4a8_status;

/* Group-size value that selects per-channel mode (one scale and zero per row). */
#define W4A8_GROUP_PER_CHANNEL 0

/* Group-size value that selects the non-uniform codebook mode (the
 * LUT-quantized, NormalFloat-style weights of the FLUTE page): per row the
 * level-1 int8 quantization (fp16 s1), then each int8 value replaced by the
 * code of the nearest of 16 fixed int8 levels (ties to the lower code):
 *   -119 -84 -65 -50 -37 -26 -15 -5 5 15 26 37 50 65 84 119
 * (standard-normal quantiles at (i + 1/2)/16 scaled to 119).  W8^ = level[q];
 * the decode is a register table lookup.  No groups, no meta section. */
#define W4A8_CODEBOOK_NF 1

/* Shape limits.  K must be a multiple of W4A8_K_QUANTUM, N of W4A8_N_QUANTUM;
 * K <= W4A8_K_MAX keeps every int32 accumulator exact (127*128*K < 2^31).
 * g must be 32, 64 or 128 (and divide K), W4A8_GROUP_PER_CHANNEL (or K), or
 * W4A8_CODEBOOK_NF. */
#define W4A8_K_QUANTUM 128
#define W4A8_N_QUANTUM 16
#define W4A8_K_MAX 131072

/* Upper bounds on the other sizes, so that every launch's grid and every
 * index fits its integer type: tokens m <= W4A8_M_MAX (and output columns
 * n <= W4A8_N_MAX) in every entry point, and rows of at most
 * W4A8_ACT_K_MAX values in the activation quantizers.  Larger sizes are
 * rejected (INVALID_ARGUMENT for m and the quantizers' k, UNSUPPORTED for n). */
#define W4A8_M_MAX (1 << 22)
#define W4A8_N_MAX (1 << 22)
#define W4A8_ACT_K_MAX (1 << 30)

/* Upper bound on the row strides of the activations the GEMM entry points
 * read (lda8 of the int8 A8, lda of the fp16 A), in elements.  The tiled
 * kernels address a 256-row activation tile through one buffer descriptor
 * with a 32-bit range; larger strides are rejected with INVALID_ARGUMENT. */
#define W4A8_LD_MAX (1 << 22)

const char* w4a8_status_string(w4a8_status s);

/* Text of the HIP error behind the most recent W4A8_ERR_DEVICE returned to
 * the calling thread ("no error" if there was none).  Static storage. */
const char* w4a8_last_device_error(void);

/* ------------------------------------------------------------------ packing
 * Packed weight blob ("layout v1").  A 256-byte header (magic, version, n, k,
 * g) is followed by three sections at offsets that depend only on (n, k, g):
 *   q     N*K/2 bytes: uint4 codes in the gfx950 register order.  For output
 *         column tile t (16 rows of W) and k-block b (128 k), 1 KiB holds, for
 *         lane l = 0..63, 16 bytes covering row 16t + (l % 16) and
 *         k = 128b + 64h + 16(l / 16) + j  (h = 0,1; j = 0..15): dword 2h
 *         holds j = 0..7, dword 2h+1 holds j = 8..15, and within a dword
 *         byte i carries j = i (low nibble) and j = i + 4 (high nibble).
 *   meta  N*G4 bytes, G4 = (groups per row) rounded up to a multiple of 4:
 *         row n holds one byte per group (low nibble z, high nibble s2 - 1)
 *         at n*G4 + group; padding bytes are 0.  Per-channel mode: 1 group.
 *         Codebook mode: empty (the header holds the 16 levels at byte 56).
 *   s1    N fp16 row scales.
 * The blob is position independent: copy it verbatim to device memory and
 * pass that copy to w4a8_gemm.  Device code never reads the header.       */

/* Bytes of the blob for (n, k, g); 0 if the shape is unsupported.  (The
 * blob layout above; the quantization it stores is w4a8_pack's.) */
size_t w4a8_packed_size(int n, int k, int g);

/* Quantize W (n x k fp32, row stride ldw >= k elements) and write the blob.
 * Defining passages: the progressive quantization of the QServe/QoQ abstract
 * (read as: weights first to int8 per output channel, then to 4 bits per
 * group, so that dequantization in the W4A8 GEMM is cheap integer work), and
 * the offline weight reordering of the same abstract (compute-aware
 * reordering), the QUICK abstract (interleaving that skips the shared-memory
 * write-back after dequantization) and the FLUTE page ("方法详解"): the codes
 * are stored in the order the matrix-core operand wants them, so the kernel
 * never rearranges them through shared memory.
 * Host only, synchronous, thread-safe.  n_threads <= 0 uses all hardware
 * threads; the output bytes do not depend on the thread count.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED, BUFFER_TOO_SMALL, NONFINITE, RANGE. */
w4a8_status w4a8_pack(const float* w, int n, int k, int ldw, int g,
                      void* blob, size_t blob_bytes, int n_threads);

/* Read (n, k, g) from a blob header (g is reported as W4A8_GROUP_PER_CHANNEL
 * in per-channel mode).  Errors: INVALID_ARGUMENT, LAYOUT. */
w4a8_status w4a8_blob_info(const void* blob, size_t blob_bytes,
                           int* n, int* k, int* g);

/* Decode a host blob back to logical arrays (for checking): q[n*k] codes,
 * z[n*G] and s2[n*G] per group (G = k/g, or 1 per channel, or 0 in codebook
 * mode: nothing written), s1[n] fp16 bits.  Any output pointer may be NULL
 * to skip it.  Errors: INVALID_ARGUMENT, LAYOUT. */
w4a8_status w4a8_unpack(const void* blob, size_t blob_bytes,
                        uint8_t* q, uint8_t* z, uint8_t* s2, uint16_t* s1);

/* ----------------------------------------------------- activation quantizer
 * Per-token int8 quantization of A (m x k fp16, row stride lda elements) into
 * a8_dev (m x k int8, row stride lda8 bytes) and s_a_dev (m fp16 scales).
 * Defining passages: the 8-bit activations of the QServe/QoQ abstract, with
 * the per-token dynamic scale that the PrefixQuant page ("Key Findings")
 * names as the usual practice.
 * m == 0 is a no-op.  k is any size from 1 to W4A8_ACT_K_MAX.  NaN/inf inputs give
 * unspecified outputs (no device-side check).
 * Errors: INVALID_ARGUMENT (null pointer, m < 0, k <= 0, lda < k, lda8 < k,
 * m > W4A8_M_MAX, k > W4A8_ACT_K_MAX), DEVICE. */
w4a8_status w4a8_quant_act(const uint16_t* a_dev, int m, int k, int lda,
                           int8_t* a8_dev, int lda8, uint16_t* s_a_dev,
                           void* stream);

/* Static per-tensor variant (the static alternative to per-token scaling on
 * the PrefixQuant page, "Key Findings"): one fp16 scale for the whole tensor,
 * fixed ahead of time, so no reduction runs.
 *   A8 = clamp(rint(A * fp32(1 / scale)), +-127)  (0 when scale == 0)
 *   s_a_dev[m] = scale for every row, so w4a8_gemm consumes it unchanged.
 * scale_f16 is the fp16 bit pattern of a finite value >= 0.  Layouts as for
 * w4a8_quant_act.  Errors: INVALID_ARGUMENT (as w4a8_quant_act, or a negative,
 * infinite or NaN scale), DEVICE. */
w4a8_status w4a8_quant_act_static(const uint16_t* a_dev, int m, int k, int lda,
                                  uint16_t scale_f16, int8_t* a8_dev, int lda8,
                                  uint16_t* s_a_dev, void* stream);

/* -------------------------------------------------------------- W4A8 GEMM
 * Y = fp16(s_a[m] * s1[n] * sum_k A8[m,k] * W8^[n,k]) with int32 accumulation.
 * Defining passages: the QServe/QoQ abstract (the int8 product runs on the
 * matrix cores and no partial sum is dequantized), and the LiquidGEMM page
 * ("Метод": each 4-bit weight is decoded to int8 in registers by a few
 * integer instructions that cannot overflow, feeding the int8 MMA directly).
 * Small M streams the weights (the FLUTE page's small-batch regime, abstract:
 * moving weights from global memory dominates); large M is bound by the
 * int8 matrix cores, the regime of the kernel speedups the LiquidGEMM page
 * reports ("Результаты").
 *   a8_dev    m x k int8, row stride lda8 bytes (k <= lda8 <= W4A8_LD_MAX,
 *             lda8 % 16 == 0, 16-byte aligned)
 *   s_a_dev   m fp16 per-token scales
 *   blob_dev  device copy of a w4a8_pack blob for (n, k, g)
 *   y_dev     m x n fp16 output, row stride ldy elements (ldy >= n)
 *   acc_dev   optional (may be NULL): m x n int32 raw accumulators, row
 *             stride ldacc elements (ldacc >= n)
 *   workspace_dev / workspace_bytes: 16-byte aligned device scratch of at
 *             least w4a8_gemm_workspace_size(m, n, k, g, opts) bytes (the
 *             same opts); may be NULL when that size is 0.  Owned by the
 *             caller; it needs no initialisation, the call overwrites it,
 *             and two calls in flight at once need two workspaces.
 *   opts      NULL for the automatic choice; otherwise forces the kernel
 *             variant and its split of K (tests and sweeps only).  Results
 *             are identical for every choice: integer partial sums are
 *             added exactly.
 * m == 0 is a no-op.  Errors: INVALID_ARGUMENT, UNSUPPORTED (k % 128, n % 16,
 * k > W4A8_K_MAX, bad g), BUFFER_TOO_SMALL, DEVICE. */
typedef struct {
  int variant;   /* 0 auto, 1 skinny (intra-workgroup split-K), 2 tiled;
                    w4a8_linear only: 3 fused quantization + skinny */
  int k_split;   /* skinny: waves that split K inside a workgroup (1..8);
                    tiled: wave groups that split the k-blocks inside a
                    workgroup (1, or 2: m_tiles x n_tiles 8 x 4 or 4 x 4
                    with 2 stages, 8 x 2 with 2-3, 4 x 2 with 2-4);
                    0 = auto */
  int n_tiles;   /* 16-column tiles per wave: skinny 1, 2 or 4; tiled 2 or 4; 0 = auto */
  int m_tiles;   /* tiled: 16-row tiles per wave (4 or 8), 0 = auto */
  int stages;    /* tiled: LDS pipeline stages, 0 = auto; four-wave tiles
                    (m_tiles x n_tiles) 8 x 4: 2-4, 4 x 4: 2-5, 8 x 2: 2-6,
                    4 x 2: 2, 3, 4, 6 or 8; eight-wave tiles as below */
  int row_groups;/* tiled: waves along M per workgroup: 1 (4 waves) or 2
                    (8 waves, 256 x 256 tiles, m_tiles 8 and 3 stages only),
                    0 = auto */
  int slices;    /* tiled: workgroups that split K of one tile (1..16), their
                    int32 partial sums going through the workspace, which
                    must then hold slices * m * n * 4 bytes; 0 = auto */
  int workgroups;/* w4a8_linear's fused kernel: workgroups of its persistent
                    grid, each walking column-tile groups (1 .. the number of
                    groups; larger values are clamped), 0 = auto */
} w4a8_gemm_opts;

/* Workspace bytes w4a8_gemm needs for these arguments (0 when it needs none,
 * or when the shape is not supported).  Host only, no HIP call. */
size_t w4a8_gemm_workspace_size(int m, int n, int k, int g, const w4a8_gemm_opts* opts);

w4a8_status w4a8_gemm(const int8_t* a8_dev, int lda8, const uint16_t* s_a_dev,
                      int m, const void* blob_dev, int n, int k, int g,
                      uint16_t* y_dev, int ldy, int32_t* acc_dev, int ldacc,
                      void* workspace_dev, size_t workspace_bytes,
                      const w4a8_gemm_opts* opts, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): w4a8_gemm
 * with no workspace argument.  When the plan splits K over workgroups, the
 * int32 partial sums go to one static device array of W4A8_SCRATCH_BYTES
 * that the library holds on each GPU it runs on until the process ends;
 * nothing is allocated or freed by the call.
 *   - Arguments and results are as for w4a8_gemm (bit-identical outputs).
 *   - The automatic plan narrows its K split until the partial sums
 *     (slices * m * n * 4 bytes) fit the array; a split forced through
 *     opts->slices that does not fit returns W4A8_ERR_BUFFER_TOO_SMALL.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents (nothing in it needs to start at zero).  Calls that
 *     overlap in time on one GPU (other streams, other threads) race on it:
 *     order them on one stream.
 *   - The first call on each device looks the array's address up
 *     (hipGetSymbolAddress, a host-side query); make that first call
 *     outside stream capture.
 * m == 0 is a no-op.  Errors as w4a8_gemm. */
#define W4A8_SCRATCH_BYTES (64u << 20)
w4a8_status w4a8_gemm_noalloc(const int8_t* a8_dev, int lda8, const uint16_t* s_a_dev,
                              int m, const void* blob_dev, int n, int k, int g,
                              uint16_t* y_dev, int ldy, int32_t* acc_dev, int ldacc,
                              const w4a8_gemm_opts* opts, void* stream);

/* ------------------------------------------------------------ whole layer
 * The W4A8 linear layer from fp16 activations: per-token quantization of A
 * (as w4a8_quant_act) followed by the GEMM (as w4a8_gemm), with A8 and s_a
 * written to a8_dev / s_a_dev as well.  Defining passage: the W4A8 layer of
 * the QServe/QoQ abstract, 8-bit activations included; fusing the
 * quantization into the small-M GEMM is this library's choice (it saves a
 * launch where the whole GEMM takes a few microseconds).  For up to 57344 activations
 * (m * k; e.g. up to 14 tokens at k = 4096, 4 at k = 14336), or 65536 on
 * layers of at least 16384 columns, both steps run in one kernel:
 * each workgroup of a persistent grid quantizes the rows itself while its
 * first weight loads are in flight, then walks several column tiles, which
 * saves a launch and a round trip of A8 through memory; otherwise it makes
 * the two calls in order on `stream`.  (opts->variant = 3 forces the fused
 * kernel for up to 16 tokens, when m rounded up to a power of two times the
 * 128-k blocks of each wave's K range is at most 64, each wave's range at
 * most 16 blocks; opts->workgroups sets its grid.)
 * Outputs are bit-identical either way (Y to the last bit: the same int32
 * sums, scales and epilogue).
 *   a_dev     m x k fp16, row stride lda elements (k <= lda <= W4A8_LD_MAX,
 *             lda % 8 == 0, 16-byte aligned)
 *   a8_dev, s_a_dev   outputs, as w4a8_quant_act (k <= lda8 <= W4A8_LD_MAX,
 *             lda8 % 16 == 0, 16-byte aligned)
 *   other arguments as w4a8_gemm; opts->variant may also be 3 to force the
 *   fused kernel (UNSUPPORTED where it does not apply); the workspace is the
 *   one w4a8_gemm_workspace_size gives for the same arguments.
 * m == 0 is a no-op.  Errors as w4a8_gemm. */
w4a8_status w4a8_linear(const uint16_t* a_dev, int lda, int m, int k,
                        const void* blob_dev, int n, int g, uint16_t* y_dev, int ldy,
                        int8_t* a8_dev, int lda8, uint16_t* s_a_dev,
                        int32_t* acc_dev, int ldacc, void* workspace_dev,
                        size_t workspace_bytes, const w4a8_gemm_opts* opts, void* stream);

/* ----------------------------------------------------- W4A16 comparison
 * The weight-only baseline the pages measure W4A8 against (the AWQ-style
 * W4A16 of the QServe/QoQ abstract, the mixed-precision kernels of the QUICK
 * abstract, FLUTE's weight-only GEMM), here on the same blob:
 * fp16 activations times the fp16 weights W16^[n,k] = fp16(s1[n] * W8^[n,k])
 * (one rounding), summed in fp32 on the fp16 MFMA:
 *   Y[m,n] = fp16(sum_k A[m,k] * W16^[n,k])
 * There is no activation quantization and no s_a.
 *   a_dev   m x k fp16, row stride lda elements (k <= lda <= W4A8_LD_MAX,
 *           lda % 8 == 0, 16-byte aligned); y_dev m x n fp16, row stride
 *           ldy >= n.
 *   opts    NULL for the automatic choice (the skinny kernel up to 64
 *           tokens, and up to 128 where the tiled grid would hold fewer than
 *           128 tiles; the tiled one above); variant 1 forces the skinny
 *           kernel (m <= 128; n_tiles / k_split as for the skinny W4A8
 *           kernel), variant 2 the tiled kernel (256 x 128 tiles, any m).
 * Results are within the fp32 summation bound of the exact sum, not
 * bit-exact across choices.  The codebook mode is not supported.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED (shape, codebook blob, variant 1
 * with m > 128), DEVICE. */
w4a8_status w4a16_gemm(const uint16_t* a_dev, int lda, int m, int k,
                       const void* blob_dev, int n, int g, uint16_t* y_dev, int ldy,
                       const w4a8_gemm_opts* opts, void* stream);

/* Kernel launches w4a8_linear makes for these arguments: 1 (fused), 2
 * (quantizer + GEMM) or 3 (quantizer + GEMM split over K + reduction); 0 if
 * the call would be rejected.  Host only, no HIP call. */
int w4a8_linear_launches(int m, int n, int k, int g, const w4a8_gemm_opts* opts);

/* ------------------------------------------------------- measurement aid
 * Not part of the layer.  A read-only stream over `bytes` of device memory
 * (16-byte aligned, a multiple of 16) by `workgroups` x 512 threads, with
 * four non-temporal 16-byte loads in flight per thread: the practical HBM
 * read ceiling that the weight-streaming regime (the FLUTE page, abstract:
 * at small batch, moving the weights from global memory dominates) is
 * measured against.  sink_dev holds `workgroups` uint32 values that are
 * written only in the rare case a workgroup's folded value equals a fixed
 * constant (so the loads cannot be optimised away); their contents mean
 * nothing.  bytes == 0 is a no-op.
 * Errors: INVALID_ARGUMENT (null pointer, misaligned or ragged size,
 * workgroups outside 1..65536), DEVICE. */
w4a8_status w4a8_read_probe(const void* src_dev, size_t bytes, int workgroups,
                            uint32_t* sink_dev, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A8_H */
