/*
 * lat_moe.h -- C ABI of the quantized latent-MoE expert stage for MI355X (gfx950).
 *
 * The operation (page "Run Edge0-145B Q3_K on AMD HIP (Linux, gfx1100) #1",
 * section "Contents" and the lat_q3k_w11.cu commit message): for every token t
 * and each of its k routed experts e = router_idx[t][j],
 *     G, U = gate and up rows of expert e (Q3_K)  x  x[t] (q8_1),
 *            integer dots per 32-value activation block, scales folded in fp32;
 *     H    = silu(G) * U, re-rounded to q8_1 (32-value blocks);
 *     O    = down rows of expert e (IQ4_NL)  x  H, same block structure;
 *     y[t] = sum over j of router_w[t][j] * O      (j = 0 .. k-1, in order).
 * Tokens are grouped by expert on the device and each expert's weights are read
 * in place.  Block layouts are ggml's GGUF formats:
 *     Q3_K   110 B per 256 weights: hmask[32] | qs[64] | scales[12] | d (fp16)
 *     IQ4_NL  18 B per  32 weights: d (fp16) | qs[16] (4-bit table indices)
 *     q8_1    36 B per  32 values : d (fp16) | s (fp16) | qs[32] (int8)
 * q8_1 rounding rule (inputs and H): amax = max|v|, d = amax/127, id = 1/d (0 if
 * d == 0), q = round-half-away(v * id), stored d = fp16(d), s = fp16(d * sum q);
 * all in IEEE fp32.
 *
 * Memory and ownership: every array argument is device memory owned by the
 * caller (for instance a torch tensor's data pointer), 16-byte aligned.  Shape
 * structs and the debug struct are host memory, read during the call only.
 * The library allocates nothing inside a call and keeps no state between calls
 * except a per-device "is this a gfx950" cache.
 *
 * Execution: work is enqueued on `stream` (a hipStream_t; NULL = the default
 * stream) and the call returns without synchronising; results are valid once
 * the stream reaches that point.  Calls that share a workspace must not
 * overlap in time.
 *
 * Errors: the return value is 0 or a LAT_MOE_E* code; nothing is enqueued when
 * an argument or workspace error is returned (these checks make no HIP call).
 * Expert ids outside [0, E) are dropped on the device: the pair contributes
 * nothing (as a zero router weight would) and is counted in the debug struct.
 */
#ifndef LAT_MOE_H
#define LAT_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LAT_MOE_OK 0
#define LAT_MOE_EINVAL 1     /* null pointer, unsupported shape, misaligned pointer */
#define LAT_MOE_EWORKSPACE 2 /* workspace_bytes smaller than lat_moe_workspace_size() */
#define LAT_MOE_EDEVICE 3    /* current device is not a gfx950 (MI355X/MI350X) */
#define LAT_MOE_ELAUNCH 4    /* a kernel launch failed (hipGetLastError after enqueue) */
#define LAT_MOE_ESCRATCH 5   /* the shapes need more workspace than LAT_MOE_NOALLOC_SCRATCH_BYTES */

#define LAT_MOE_MAX_E 1024
#define LAT_MOE_ROUTER_MAX_E 1024 /* experts the router takes */
#define LAT_MOE_ROUTER_MAX_K 64   /* picks per token the router takes */

/* Shapes of one call.  Supported: T >= 0, T * k < 2^31, L % 256 == 0
 * (256 <= L <= 65536), F % 32 == 0 (32 <= F <= 65536), 1 <= E <= 1024,
 * 1 <= k <= E, T * L < 2^31, T * k * F < 2^31, and one expert's weights
 * below 2 GiB (2F * L/256 * 110 and L * F/32 * 18 bytes < 2^31). */
typedef struct lat_moe_shapes {
  int64_t T; /* tokens */
  int32_t L; /* latent dimension */
  int32_t F; /* expert FFN width */
  int32_t E; /* experts */
  int32_t k; /* experts per token */
} lat_moe_shapes;

/* Bytes of device workspace lat_moe_expert_forward needs for these shapes
 * (0 if the shapes are unsupported).  Grows with T*k*(F + 4L). */
size_t lat_moe_workspace_size(const lat_moe_shapes* shapes);

/* The expert stage.
 *   x_q8_1      [T][L/32] q8_1 blocks         latent activations, already in q8_1
 *   router_idx  [T][k] int32                  routed expert ids
 *   router_w    [T][k] fp32                   combine weights, used as given
 *   gateup_q3k  [E][2F][L/256] Q3_K blocks    rows 0..F-1 gate, F..2F-1 up
 *   down_iq4nl  [E][L][F/32] IQ4_NL blocks
 *   y           [T][L] fp32                   output, overwritten
 *   workspace   workspace_bytes of device memory, contents need no initialisation
 *   stream      hipStream_t
 * Results are deterministic: the same inputs give bitwise identical y. */
int lat_moe_expert_forward(const void* x_q8_1, const int32_t* router_idx, const float* router_w,
                           const void* gateup_q3k, const void* down_iq4nl, const lat_moe_shapes* shapes,
                           float* y, void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the expert
 * stage of lat_moe_expert_forward (same arguments without the workspace,
 * same kernels, same y bit for bit), its workspace taken from a device array
 * of LAT_MOE_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it
 * runs on until the process ends.  Shapes whose lat_moe_workspace_size
 * exceeds that return LAT_MOE_ESCRATCH (nothing enqueued); with L = 1024,
 * F = 2048 and k = 8 that is above about 1300 tokens.  The call allocates
 * nothing.  All calls on one GPU share its array: calls that overlap in time
 * on one GPU (other streams, other threads) race, and must be serialised by
 * the caller. */
#define LAT_MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int lat_moe_expert_forward_noalloc(const void* x_q8_1, const int32_t* router_idx, const float* router_w,
                                   const void* gateup_q3k, const void* down_iq4nl, const lat_moe_shapes* shapes,
                                   float* y, void* stream);

/* Options and optional device outputs of lat_moe_expert_forward_ex.  Any
 * pointer may be NULL.  A zero-filled struct asks for no debug output and
 * for the combine by atomic adds (deterministic = 0). */
typedef struct lat_moe_debug {
  void* h_q8_1;         /* [T*k][F/32] q8_1: H of every pair p = t*k + j, ggml layout;
                           pairs with an invalid expert id get all-zero blocks */
  int32_t* perm;        /* [T*k]: pair ids grouped by expert, ascending within an expert;
                           only the first offsets[E] entries are defined */
  int32_t* offsets;     /* [E+1]: start of each expert's group in perm */
  int32_t* dropped;     /* [1]: number of pairs whose expert id is outside [0, E) */
  /* Integer block dots as the kernels form them, for a range of weight rows:
   * gateup_i32 [T*k][gu_rows][L/32] for gate/up rows gu_row0 .. gu_row0+gu_rows-1
   * (of 2F), each the dot of the scale-folded Q3_K row with the token's q8_1
   * codes over one 32-value block: sum sigma(i/16) * (c(i) - 4) * q(i).
   * down_i32 [T*k][dn_rows][F/32] for down rows dn_row0 .. dn_row0+dn_rows-1
   * (of L): sum over a block of table(idx(i)) * qH(i).  Entries of invalid
   * pairs are left untouched. */
  int32_t* gateup_i32;
  int32_t gu_row0, gu_rows;
  int32_t* down_i32;
  int32_t dn_row0, dn_rows;
  /* Five caller-created hipEvent_t handles (timing enabled), recorded on
   * `stream` before the route kernels, after them, after gate/up, after down
   * and after the combine, so elapsed times between consecutive events are the
   * stage durations.  NULL to skip.  Recording adds no kernel. */
  void* const* stage_events;
  /* How the k expert outputs of a token are summed into y (the weighted
   * combine; the pages do not say):
   *   nonzero  each pair's weighted row goes to a slot of the workspace and a
   *            combine kernel adds a token's slots in slot order j = 0..k-1:
   *            the same inputs give bitwise identical y (what
   *            lat_moe_expert_forward does);
   *   0        the down kernel adds each weighted row into y with fp32 atomic
   *            adds (y is zeroed by the route pass): no slot buffer and no
   *            combine kernel, but the order of the k additions, and so the
   *            rounding of y, may change from call to call.
   * Batches of at most 64 pairs (L <= 1024, F <= 2048) sum a token's experts
   * in slot order inside the down kernel either way, so their y is always
   * deterministic. */
  int32_t deterministic;
} lat_moe_debug;

/* The expert stage with options and debug outputs: the arguments and rules of
 * lat_moe_expert_forward, plus dbg (host memory, may be NULL: then the call is
 * lat_moe_expert_forward).  Debug row ranges must lie inside [0, 2F) and
 * [0, L); stage_events, when given, must hold five non-NULL events. */
int lat_moe_expert_forward_ex(const void* x_q8_1, const int32_t* router_idx, const float* router_w,
                              const void* gateup_q3k, const void* down_iq4nl, const lat_moe_shapes* shapes,
                              float* y, void* workspace, size_t workspace_bytes, void* stream,
                              const lat_moe_debug* dbg);

/* Formats of the down weights for lat_moe_expert_forward_fmt.  Both are
 * 18-byte blocks of 32 weights, fp16 d then 16 bytes of 4-bit indices
 * (element i < 16 in the low nibble of byte i, element i >= 16 in the high
 * nibble of byte i - 16); a weight is d * K(index) with
 *   IQ4_NL: K = {-127, -104, -83, -65, -49, -35, -22, -10, 1, 13, 25, 38, 53, 69, 89, 113}
 *   Q4_0:   K(index) = index - 8
 * (ggml's block formats; Q4_0 is among the weight formats named in section
 * "Not done" of the page "Run Edge0-145B Q3_K on AMD HIP (Linux, gfx1100) #1",
 * here read as a format of the expert's down weights). */
#define LAT_MOE_DOWN_IQ4_NL 0
#define LAT_MOE_DOWN_Q4_0 1

/* Formats of the gate/up weights for lat_moe_expert_forward_fmt:
 *   LAT_MOE_GATEUP_Q3_K  [E][2F][L/256] Q3_K super-blocks (110 B), as above;
 *   LAT_MOE_GATEUP_Q4_0  [E][2F][L/32] Q4_0 blocks (18 B, the layout above,
 *                        weight = d * (nibble - 8)), one scale per 32 values:
 *                        G/U = sum over blocks of d_w * d_x * I32, with I32
 *                        the int32 dot of the nibble - 8 values and the
 *                        activation codes (the gateup_i32 probe). */
#define LAT_MOE_GATEUP_Q3_K 0
#define LAT_MOE_GATEUP_Q4_0 1

/* The expert stage with a choice of weight formats: gateup is [E][2F][...]
 * blocks of gateup_format and down [E][L][F/32] blocks of down_format (any
 * other value returns LAT_MOE_EINVAL).  Every other argument, rule and result
 * is that of lat_moe_expert_forward_ex (with Q4_0 gate/up weights one expert's
 * 2F * L/32 * 18 bytes must stay below 2^31); dbg may be NULL, and its probes
 * hold the formats' integer dots.  With LAT_MOE_GATEUP_Q3_K and
 * LAT_MOE_DOWN_IQ4_NL the call is lat_moe_expert_forward_ex. */
int lat_moe_expert_forward_fmt(const void* x_q8_1, const int32_t* router_idx, const float* router_w,
                               const void* gateup, int32_t gateup_format, const void* down, int32_t down_format,
                               const lat_moe_shapes* shapes, float* y, void* workspace, size_t workspace_bytes,
                               void* stream, const lat_moe_debug* dbg);

/* Round fp32 rows to q8_1 with the rule above: x [rows][cols] -> out
 * [rows][cols/32] q8_1 blocks (cols % 32 == 0, rows >= 0).  This is the rounding
 * the stage's producer applies to the latent rows (the D projection's q8_1
 * store) and the same rule the stage applies to H. */
int lat_moe_quantize_q8_1(const float* x, int64_t rows, int32_t cols, void* out_q8_1, void* stream);

/* Latent D / U dense projection (page "Run Edge0-145B Q3_K on AMD HIP (Linux,
 * gfx1100) #1", the lat_dense_w11.cu commit message: the two dense projections
 * of a latent layer, D into the latent rows and U back out of them, as Q8_0 x
 * q8_1 integer dots; D stores its products as the latent rows' q8_1 blocks):
 *     y[t][n] = sum over 32-value blocks b of d_w[n][b] * d_x[t][b] * I[t][n][b],
 *     I[t][n][b] = sum over the block of qw * qx   (int32, exact),
 * scales folded in fp32.
 *   x_q8_1   [T][K/32] q8_1 blocks            activations
 *   w_q8_0   [N][K/32] Q8_0 blocks, 34 B each: d (fp16) | qs[32] (int8)
 *   y_f32    [T][N] fp32, overwritten, or NULL
 *   y_q8_1   [T][N/32] q8_1 blocks, overwritten, or NULL: y rounded with the
 *            q8_1 rule above (the same bytes lat_moe_quantize_q8_1 makes of y_f32)
 *   stream   hipStream_t
 * Supported: T >= 0, K % 32 == 0, N % 32 == 0, 32 <= K, N <= 65536,
 * N * K/32 * 34 < 2^31 and T * K/32 * 36 < 2^31 bytes.  At least one output
 * must be given; pointers 16-byte aligned (the weight rows themselves are only
 * 2-byte aligned and are read as such).  T = 0 enqueues nothing.  Outputs are
 * deterministic.  No workspace.  For T <= 8, a call with y_f32 given spreads
 * the weight rows over many more workgroups (and, if y_q8_1 is given too,
 * rounds y_f32 in a second kernel); with y_q8_1 alone one workgroup takes
 * each 32 rows, which is slower for few rows.  The bytes are the same. */
int lat_moe_dense_q8_0(const void* x_q8_1, const void* w_q8_0, int64_t T, int32_t N, int32_t K, float* y_f32,
                       void* y_q8_1, void* stream);

/* As lat_moe_dense_q8_0, plus the integer block dots I of weight rows
 * row0 .. row0+rows-1: dots_i32 [T][rows][K/32] int32 (device memory);
 * 0 <= row0, 1 <= rows, row0 + rows <= N. */
int lat_moe_dense_q8_0_debug(const void* x_q8_1, const void* w_q8_0, int64_t T, int32_t N, int32_t K,
                             float* y_f32, void* y_q8_1, void* stream, int32_t* dots_i32, int32_t row0,
                             int32_t rows);

/* The same projection with Q4_0 weights: w_q4_0 [N][K/32] blocks of 18 B,
 * d (fp16) | qs[16], element i < 16 the low nibble of qs[i], element i >= 16
 * the high nibble of qs[i - 16], weight = d * (nibble - 8) (ggml's Q4_0; the
 * page "Run Edge0-145B Q3_K on AMD HIP (Linux, gfx1100) #1", section "Not
 * done", names a Q4_0 projection file).  I is then the int32 dot of the
 * nibble - 8 values with the activation codes.  Rules, outputs and errors as
 * for lat_moe_dense_q8_0, with N * K/32 * 18 < 2^31 bytes of weights and one
 * more shape rule: T <= 8 (and K <= 4096, or K <= 8192 with T <= 4), or
 * N % 128 == 0 and K % 256 == 0; other shapes return LAT_MOE_EINVAL. */
int lat_moe_dense_q4_0(const void* x_q8_1, const void* w_q4_0, int64_t T, int32_t N, int32_t K, float* y_f32,
                       void* y_q8_1, void* stream);

/* As lat_moe_dense_q4_0, plus the integer block dots of weight rows
 * row0 .. row0+rows-1, as for lat_moe_dense_q8_0_debug. */
int lat_moe_dense_q4_0_debug(const void* x_q8_1, const void* w_q4_0, int64_t T, int32_t N, int32_t K,
                             float* y_f32, void* y_q8_1, void* stream, int32_t* dots_i32, int32_t row0,
                             int32_t rows);

/* Router (page "Run Edge0-145B Q3_K on AMD HIP (Linux, gfx1100) #1", section
 * "Contents", and the HIP backend page: each token's top experts and the
 * weights the stage combines their outputs with): softmax of each token's
 * logits over the E experts, the k largest probabilities in descending order
 * (equal logits: ascending expert id), the k probabilities renormalised to
 * sum to one.  Computed as the softmax of the k picked logits (the full
 * denominator cancels; softmax ranks as the logits do), in fp32.
 *   logits      [T][E] fp32; every row needs a finite maximum; -inf marks an
 *               expert no token may prefer (picked only when fewer than k
 *               logits of the row are finite, then with weight 0); NaN is
 *               not supported
 *   router_idx  [T][k] int32 out, router_w [T][k] fp32 out: the stage's inputs
 * Supported: T >= 0, 1 <= E <= LAT_MOE_ROUTER_MAX_E, 1 <= k <= min(E,
 * LAT_MOE_ROUTER_MAX_K); pointers 16-byte aligned.  T = 0 enqueues nothing. */
int lat_moe_router_topk(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* router_idx, float* router_w,
                        void* stream);

/* Static description of an error code. */
const char* lat_moe_strerror(int code);

/* Library version: major * 10000 + minor * 100 + patch. */
int lat_moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LAT_MOE_H */
