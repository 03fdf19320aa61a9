/*
 * oft.h -- C ABI of liboft: the OFT-adapted linear layer over a frozen
 * low-precision base, and its MoE (grouped, active-expert) form, for AMD
 * Instinct MI355X (gfx950).
 *
 * Method (sources are the Orbit pages):
 *   - Sphere AI Lab's Orbit release news (chooseai.io), section "Technical
 *     principles": the base stays frozen at deployment precision (INT4/FP8)
 *     and every gradient goes through a small BF16 OFT adapter;
 *   - same page, "Five design features of the adapter-first architecture"
 *     and "Architectural advantages of OFT over LoRA": each sub-projection of
 *     a fused tensor (Q/K/V, gate/up) gets its own orthogonal rotation;
 *   - same page, "Dedicated optimisation for low-precision MoE models", and
 *     the Synced article on Orbit, section "Technical details": only the
 *     router-selected experts are dequantised, in fixed-size batches, before
 *     a grouped GEMM; the backward never computes a base-weight gradient.
 *   The pages print no formula.  This library implements: each output
 *   channel block j (b consecutive channels; segments are multiples of b)
 *   has R_j = (I + Q_j)(I - Q_j)^-1 with Q_j skew-symmetric, and
 *   y = rot_R(x . dequant(W0)^T), i.e. Y[:, blk j] = Z[:, blk j] . R_j^T
 *   with Z = x . dequant(W0)^T.  Training produces dX and dQ only.
 *
 * Conventions shared by every entry point
 *   - Every tensor argument is a caller-owned DEVICE pointer, 16-byte
 *     aligned, row-major and contiguous.  Descriptors (structs passed by
 *     pointer) are HOST memory, read only during the call.
 *   - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *     A call validates its arguments on the host, enqueues kernels on
 *     `stream` and returns; it never synchronises and never allocates.
 *     Scratch memory is the caller's workspace `ws` of `ws_bytes` bytes,
 *     sized by the matching *_workspace_bytes query.
 *   - Return value: OFT_OK or a negative oft_status.  On every error except
 *     OFT_EHIP nothing has been enqueued and no output was touched.
 *     OFT_EHIP means a launch failed; oft_last_hip_error() returns the
 *     hipError_t (thread-local).  Faults inside kernels surface at the
 *     caller's next synchronisation.
 *   - Results are deterministic: no floating-point atomics; every reduction
 *     runs in a fixed order.  Calls are re-entrant; calls on different
 *     streams may overlap only if they share no output or workspace.
 *   - Encodings: bf16 / fp16 tensors are uint16_t bit patterns; fp8 is OCP
 *     e4m3fn (bias 7, max 448, no infinities).  INT4 weights are uint8
 *     [rows, cols/2]: element c of a row sits in byte c/2, low nibble for
 *     even c, two's complement in [-8, 7]; INT4 scales are fp16
 *     [rows, cols/g] (group of g consecutive in-features).  FP8 weights are
 *     uint8 [rows, cols] with fp32 scales [rows] (one per output channel).
 *   - Adapter parameters q: bf16 [nblk, b(b-1)/2], the strict upper triangle
 *     of each Q_j in row-major order (0,1),(0,2),...,(0,b-1),(1,2),...;
 *     entry p of pair (i,l) sets Q[i][l] = p and Q[l][i] = -p.  Block j
 *     covers output channels [j*b, (j+1)*b).
 *   - Rotation operand R_ops: bf16 [nblk, 2, b, b]; [j][0] is R_j and [j][1]
 *     is R_j^T (both row-major).  R_f32: fp32 [nblk, b, b], R_j row-major.
 */
#ifndef OFT_H_
#define OFT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OFT_ABI_VERSION 8

typedef enum {
  OFT_OK = 0,
  OFT_EINVAL = -1,      /* null required pointer, bad size, misaligned pointer */
  OFT_ESHAPE = -2,      /* shape constraint violated (see each call)           */
  OFT_EDTYPE = -3,      /* unknown dtype / format enum                          */
  OFT_EUNSUPPORTED = -4,/* valid but not implemented (b, g, k, segments)        */
  OFT_EWORKSPACE = -5,  /* workspace smaller than the query returned            */
  OFT_EHIP = -6         /* a HIP launch failed; see oft_last_hip_error()        */
} oft_status;

enum { OFT_DT_BF16 = 0, OFT_DT_F32 = 1 };
/* OFT_W_BF16: weights already dequantised to bf16 (MoE calls only; the
 * dense-weight reference that the grouped dequant GEMMs are measured
 * against: same kernels, no scales, two bytes per weight in HBM). */
/* OFT_W_FP4_E2M1: an FP4 base (the chooseai.io page's "Technical
 * principles" section lists FP4 among the frozen base precisions, and the
 * Synced article's DeepSeek V4 Flash experiment trains a BF16 adapter on an
 * FP4 base) in the OCP Microscaling form: E2M1 codes
 * (1 sign, 2 exponent bits with bias 1, 1 fraction bit; 0, 0.5, 1, 1.5, 2,
 * 3, 4, 6 and their negatives), two per byte, low nibble first, exactly as
 * INT4 codes; one scale slot per group of g codes along K, also as INT4, but
 * each 16-bit slot holds an E8M0 exponent code c in its low byte (the high
 * byte is ignored): w = e2m1(code) * 2^(c - 127).  g = 32 is the OCP MXFP4
 * block; its one-byte scales are widened to 16 bits.  c = 255 (NaN in the
 * OCP format) is not supported: its results are unspecified. */
/* OFT_W_INT4_TILED (MoE calls only): the INT4 weights of OFT_W_INT4 (same
 * values, same fp16 group scales: the frozen 4-bit base of the QOFT paper's
 * "Quantized OFT" section) with each expert matrix [N, K] stored in tiles of
 * 64 rows x 128 columns, tile (rb, kb) the (rb * K/128 + kb)-th: codes 4096
 * bytes a tile, the tile's row r at byte 64 r (its 128 codes as in a
 * row-major row); scales 16384/g bytes a tile, the tile's row r at byte
 * r 256/g (its 128/g slots in column order).  The arrays have the sizes of
 * the row-major ones; oft_pack_int4_tiled converts.  The grouped GEMMs then
 * read each 64-row block's codes and scales for a K step as contiguous
 * runs. */
enum { OFT_W_INT4 = 0, OFT_W_FP8_E4M3 = 1, OFT_W_BF16 = 2, OFT_W_FP4_E2M1 = 3, OFT_W_INT4_TILED = 4 };
enum { OFT_PASS_FWD = 0, OFT_PASS_BWD = 1 };

#define OFT_MAX_SEGMENTS 8

/* Dense OFT linear layer: x [M, K] -> y [M, N], N = sum(seg).
 * Constraints: M >= 0 (M == 0 is a no-op); K >= 64 and K % 64 == 0;
 * b in {16, 32}; 1 <= n_seg <= 8, every seg[s] > 0 and seg[s] % b == 0,
 * N % 32 == 0; INT4 and FP4: g in {32, 64, 128} and K % g == 0.
 * Size range (else OFT_EUNSUPPORTED): M <= 2^22, K and N <= 2^20 and
 * N * K < 2^31 (token tiles run along the launch grid's y dimension, and
 * weight offsets inside the kernels are 32-bit). */
typedef struct {
  int32_t M, K, N;
  int32_t x_dtype; /* OFT_DT_BF16 | OFT_DT_F32; y and dx use the same dtype */
  int32_t w_fmt;   /* OFT_W_INT4 | OFT_W_FP8_E4M3 | OFT_W_FP4_E2M1         */
  int32_t g;       /* INT4 / FP4 group size along K (ignored for FP8)      */
  int32_t b;       /* OFT block size                                       */
  int32_t n_seg;
  int32_t seg[OFT_MAX_SEGMENTS];
} oft_linear_desc;

/* MoE layer: T tokens, E experts, top-k routing, hidden H, expert
 * intermediate I.  Per expert e: gate/up weight [2I, H] (gate rows [0, I),
 * up rows [I, 2I)) with its own adapter of 2I/b blocks (gate blocks first),
 * down weight [H, I] without adapter; INT4 with group g (w_fmt =
 * OFT_W_INT4, zero, or OFT_W_INT4_TILED, the same values tiled), FP4 with
 * group g (OFT_W_FP4_E2M1, the same layout with E8M0 exponents in the scale
 * slots) or, as a measurement reference, bf16
 * (OFT_W_BF16: the
 * code arrays hold bf16 weights [E, 2I, H] and [E, H, I], the scale
 * pointers are ignored and may be NULL, g is not checked).
 * Constraints: T >= 0; 1 <= k <= 16; k <= E <= 1024; H % 64 == 0;
 * I % 64 == 0; b in {16, 32}; I % b == 0; INT4 and FP4: g in {32, 64,
 * 128}, H % g == 0, I % g == 0; OFT_W_INT4_TILED: H % 256 == 0 and
 * I % 256 == 0 (else OFT_ESHAPE); chunk >= 1; renorm in {0, 1}; w_fmt one
 * of the four formats above (else OFT_EDTYPE).  Size range (else
 * OFT_EUNSUPPORTED): H and I <= 2^16, I H < 2^31 (code offsets inside an
 * expert are 32-bit), ceil(T k / 16) + E <= 65535 (the grouped work list
 * runs along the launch grid's y dimension). */
typedef struct {
  int32_t T, E, k, H, I, g, b;
  int32_t chunk;  /* active experts per chunk (scheduling unit)            */
  int32_t renorm; /* 0: combine weights = softmax over all E at the chosen
                     experts; 1: renormalised over the k chosen             */
  int32_t w_fmt;  /* OFT_W_INT4 (0), OFT_W_INT4_TILED, OFT_W_FP4_E2M1 or
                     OFT_W_BF16                                             */
} oft_moe_desc;

/* Routing tables: device pointers, caller-allocated, written by the
 * forward (oft_moe_route / oft_moe_grouped_fwd) and read by the backward.
 * P = T*k routed (token, slot) pairs, pair id t*k + j. */
typedef struct {
  int32_t* topk_idx;        /* [T, k] expert of slot j, descending logit, ties -> lower id */
  float* topk_w;            /* [T, k] combine weights                            */
  int32_t* counts;          /* [E]    pairs per expert                           */
  int32_t* offsets;         /* [E+1]  exclusive scan of counts                   */
  int32_t* perm;            /* [P]    pos -> pair id, ordered by (expert, token)  */
  int32_t* inv_perm;        /* [P]    pair id -> pos                             */
  int32_t* active;          /* [E]    active expert ids ascending, then -1        */
  int32_t* n_active;        /* [1]                                               */
  int32_t* chunk_of_expert; /* [E]    active rank / chunk, -1 when inactive      */
} oft_moe_routing;

/* ---- helpers ------------------------------------------------------------ */
int32_t oft_abi_version(void);
const char* oft_status_str(int32_t status); /* static string, never NULL */
int32_t oft_last_hip_error(void);           /* hipError_t of the last OFT_EHIP */

/* ---- opt-in kernel timing (measurement only) ------------------------------
 * oft_prof_enable(1) clears the record list and starts recording: from then
 * on every call records, per step of its work (e.g. "moe.gateup",
 * "dense.fwd", "dense.dq"), a HIP event on its launch stream before and
 * after the kernels of that step; oft_prof_enable(0) stops recording (the
 * records stay readable) and is the default.  The first enable creates the
 * event pool (2 x 1024 events of the device current then; records past 1024
 * are dropped); recording does not allocate device memory.  oft_prof_count()
 * returns the number of records; oft_prof_read(i, ...) waits for record i's
 * second event and writes its name (NUL-terminated, truncated to name_len)
 * and its duration in milliseconds.  Process-wide, serialised by a mutex;
 * not for use during graph capture.  Errors: OFT_EINVAL (index out of
 * range, NULL output, name_len < 1), OFT_EHIP (event creation or wait). */
int32_t oft_prof_enable(int32_t on);
int32_t oft_prof_count(void);
int32_t oft_prof_read(int32_t i, char* name, int32_t name_len, float* ms);

/* ---- Cayley map (adapter -> rotation) ------------------------------------
 * Per block: A = I - Q_j, R_j = (I + Q_j) A^-1 = 2 A^-1 - I, by Gauss-Jordan
 * elimination without pivoting in fp32 (the symmetric part of A is I, so the
 * pivots stay >= 1).
 * q_bf16 [nblk, b(b-1)/2] -> R_f32 [nblk, b, b] and, when R_ops is not NULL,
 * the bf16 operand pack [nblk, 2, b, b] (R, R^T; round to nearest even).
 * nblk == 0 is a no-op.  Errors: OFT_EINVAL (null, nblk < 0),
 * OFT_EUNSUPPORTED (b not in {16, 32}). */
int32_t cayley_build(const uint16_t* q_bf16, int32_t nblk, int32_t b, float* R_f32,
                     uint16_t* R_ops_or_null, void* stream);

/* ---- dequantisation hook (what the matrix cores consume) ------------------
 * INT4: out[r][c] = bf16_RNE(q[r][c] * s[r][c / g]) (the product is exact in
 * fp32, so this is one rounding).  FP4: out[r][c] = bf16_RNE(e2m1(code) *
 * 2^(c_e - 127)) with c_e the exponent code of the group (exact short of
 * overflow).  FP8: out[r][c] = e4m3fn(code) exactly;
 * the per-row scale is NOT applied (the GEMMs apply it in fp32 outside the
 * K loop).  codes: INT4 / FP4 [rows, cols/2] / FP8 [rows, cols]; scales:
 * 16-bit [rows, cols/g] (INT4 fp16, FP4 exponent codes) / ignored for FP8
 * (may be NULL); out_bf16 [rows, cols].  Constraints: rows, cols >= 0,
 * cols % 8 == 0; INT4 and FP4: g in {32, 64, 128}, cols % g == 0. */
int32_t oft_dequant(int32_t w_fmt, int32_t rows, int32_t cols, int32_t g, const uint8_t* codes,
                    const void* scales, uint16_t* out_bf16, void* stream);

/* ---- tiled INT4 storage (see OFT_W_INT4_TILED) ----------------------------
 * Writes the tiled copy of `count` row-major INT4 weights [rows, cols] (group
 * g) stored one after another: codes [count, rows, cols/2] -> codes_tiled
 * (same size), fp16 scales [count, rows, cols/g] -> scales_tiled (same size).
 * A permutation of bytes (exact); the weights are frozen, so a caller packs
 * once, e.g. at load.  Device pointers, 16-byte aligned; the outputs may not
 * overlap the inputs.  Constraints: count, rows, cols >= 0 (a zero is a
 * no-op); rows % 64 == 0 and cols % 128 == 0 (else OFT_ESHAPE); g in {32,
 * 64, 128} (else OFT_EUNSUPPORTED); rows cols < 2^32 (else
 * OFT_EUNSUPPORTED).  Errors: OFT_EINVAL (null / misaligned / overlapping
 * pointers, negative sizes), OFT_EHIP. */
int32_t oft_pack_int4_tiled(int32_t count, int32_t rows, int32_t cols, int32_t g, const uint8_t* codes,
                            const uint16_t* scales, uint8_t* codes_tiled, uint16_t* scales_tiled, void* stream);

/* ---- dense layer ----------------------------------------------------------
 * Workspace query for `pass` (OFT_PASS_FWD / OFT_PASS_BWD); writes *bytes. */
int32_t oft_linear_workspace_bytes(const oft_linear_desc* d, int32_t pass, size_t* bytes);

/* Forward: y = rot_R(x . dequant(W0)^T).
 * x [M, K] (x_dtype), w_codes / w_scales (w_fmt layout, N rows, K cols),
 * R_ops from cayley_build, y [M, N] (x_dtype).  The dequantised tile never
 * leaves LDS; bf16 matrix-core products accumulate in fp32; the FP8 row
 * scale multiplies the fp32 accumulator; the block rotation runs in the
 * epilogue on bf16 operands with fp32 accumulation. */
int32_t oft_linear_fwd(const oft_linear_desc* d, const void* x, const uint8_t* w_codes,
                       const void* w_scales, const uint16_t* R_ops, void* y, void* ws,
                       size_t ws_bytes, void* stream);

/* ---- double-buffered adapter slots ----------------------------------------
 * The pages keep a version number per adapter and stream a new version into
 * the inactive of two slots while the active one keeps serving, then switch
 * atomically (the Synced article's "Technical details" section; the
 * chooseai.io page's "Five design features of the adapter-first
 * architecture").  The caller owns the two rotation packs R_ops0 / R_ops1
 * ([nblk, 2, b, b] bf16 each, written by cayley_build) and a device int32
 * state[2]: [0] the active slot (0 or 1), [1] the adapter version it holds,
 * kept as one 64-bit word.  Zero the state before first use (slot 0
 * active, version 0).
 *
 * oft_slots_switch: after the work enqueued before it on `stream` (the
 * Cayley build into `slot`), state = {slot, version} by one device-scope
 * atomic 64-bit store, so a reader sees the old pair or the new one, never
 * a mix.  Errors: OFT_EINVAL (state NULL or misaligned, slot not 0 or
 * 1). */
int32_t oft_slots_switch(int32_t* state, int32_t slot, int32_t version, void* stream);

/* oft_linear_fwd on the active slot.  One thread first copies {active slot,
 * its version} from state (one atomic 64-bit load) into latch (device int32[2], caller-owned), then
 * every workgroup of the forward reads latch[0]: one call uses one slot
 * throughout, and latch[1] names the adapter version that produced y.
 * Every call in flight needs a latch of its own: a later call on another
 * stream (or another branch of a graph) writing the same latch while an
 * earlier forward still reads it could switch that forward's slot midway.  The
 * slot is read when the kernels run, not when they are enqueued, so a graph
 * captured once follows every later switch.  The double buffer lets a build
 * into the inactive slot and a switch overlap with forwards on the active
 * one; a build into a slot must not overlap with a forward that latched
 * that slot (order them with an event across streams).  Workspace: none.
 * M == 0 still writes the latch.  Errors: as oft_linear_fwd, and
 * OFT_EINVAL for a NULL or misaligned state, latch, R_ops0 or R_ops1. */
int32_t oft_linear_fwd_slots(const oft_linear_desc* d, const void* x, const uint8_t* w_codes,
                             const void* w_scales, const uint16_t* R_ops0, const uint16_t* R_ops1,
                             const int32_t* state, int32_t* latch, void* y, void* ws, size_t ws_bytes,
                             void* stream);

/* Reference-policy forward: y = x . dequant(W0)^T, the frozen base alone
 * (R = I).  The pages' section "Five design features of the adapter-first
 * architecture" takes the KL reference from the frozen base without the
 * adapter, so no copy of the actor is kept; this is that layer, run by the
 * forward kernels with the rotation epilogue left out.  bf16 y is
 * bit-identical to oft_linear_fwd with Q = 0 (whose R is exactly I); fp32 y
 * is Z itself, which the adapted path rounds to bf16 for the rotation.
 * Arguments as in
 * oft_linear_fwd, without R_ops; the block size b is validated but plays no
 * part.  Workspace: none (ws may be NULL).  Errors as oft_linear_fwd. */
int32_t oft_linear_fwd_base(const oft_linear_desc* d, const void* x, const uint8_t* w_codes,
                            const void* w_scales, void* y, void* ws, size_t ws_bytes, void* stream);

/* Backward of <dy, y>: dx = rot_R^T(dy) . dequant(W0) and dq (fp32, packed
 * like q).  dy [M, N] bf16; y_saved [M, N] (x_dtype) is the forward output
 * (dq uses Z = y R recomputed from it); R_f32 / R_ops from cayley_build.
 * dx_or_null [M, K] (x_dtype) and dq_or_null [nblk, b(b-1)/2] may each be
 * NULL to skip that gradient.  No gradient of the frozen base is formed. */
int32_t oft_linear_bwd(const oft_linear_desc* d, const uint16_t* dy, const void* y_saved,
                       const uint8_t* w_codes, const void* w_scales, const float* R_f32,
                       const uint16_t* R_ops, void* dx_or_null, float* dq_or_null, void* ws,
                       size_t ws_bytes, void* stream);

/* oft_linear_bwd without a workspace, for callers that cannot allocate
 * (code under graph capture, tight serving loops, harnesses that forbid
 * allocation).  Arguments and results as oft_linear_bwd; its scratch is a
 * fixed device array of OFT_NOALLOC_SCRATCH_BYTES inside the library, held
 * by every GPU the library runs on until the process ends (looked up once
 * per device, on the first call there).  It allocates nothing and
 * synchronises nothing.  Calls that overlap on one GPU (different streams,
 * parallel graph branches) share the array and race: order them.  Errors:
 * as oft_linear_bwd, and OFT_EWORKSPACE when the layer's backward needs
 * more scratch than the array holds (oft_linear_workspace_bytes(d,
 * OFT_PASS_BWD) > OFT_NOALLOC_SCRATCH_BYTES: e.g. the 4096-token fused QKV
 * layer of a 4B model fits, the 8192-token gate/up layer does not). */
#define OFT_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int32_t oft_linear_bwd_noalloc(const oft_linear_desc* d, const uint16_t* dy, const void* y_saved,
                               const uint8_t* w_codes, const void* w_scales, const float* R_f32,
                               const uint16_t* R_ops, void* dx_or_null, float* dq_or_null, void* stream);

/* ---- reference-policy log-probabilities ------------------------------------
 * The KL regulariser of the pages compares the trained policy with the
 * frozen base run without the adapter (the chooseai.io page's "Five design
 * features of the adapter-first architecture": zero extra reference model);
 * its estimate needs both policies' log-probability of the sampled token.
 * out[t] = log softmax(logits_actor[t])[labels[t]]
 *        - log softmax(logits_ref[t])[labels[t]]   (natural log, fp32)
 * logits_* fp32 [T, V] (e.g. the vocabulary projection of the adapted layers'
 * and the oft_*_fwd_base outputs), labels int32 [T], out fp32 [T]; a label
 * outside [0, V) gives NaN.  Deterministic (fixed-order reductions).
 * T == 0 is a no-op.  Errors: OFT_EINVAL (T < 0, V < 1, T V >= 2^40, a NULL
 * or misaligned pointer). */
int32_t oft_logprob_diff(int32_t T, int32_t V, const float* logits_actor, const float* logits_ref,
                         const int32_t* labels, float* out, void* stream);

/* ---- MoE layer ------------------------------------------------------------ */
int32_t oft_moe_workspace_bytes(const oft_moe_desc* d, int32_t pass, size_t* bytes);

/* Routing only: top-k of fp32 logits [T, E] (descending, ties to the lower
 * expert id), softmax combine weights, per-expert counts, exclusive-scan
 * offsets, the stable (expert, token) permutation and its inverse, the
 * active-expert list and chunk table.  All on the device, no host sync. */
int32_t oft_moe_route(const oft_moe_desc* d, const float* logits, const oft_moe_routing* rt,
                      void* ws, size_t ws_bytes, void* stream);

/* Forward: routing (as oft_moe_route), then for the active experts, chunk by
 * chunk, the gate/up dequant grouped GEMM over the gathered token rows with
 * the per-expert split rotation in its epilogue -> h_saved [P, 2I] bf16 in
 * permuted order; SwiGLU; the down dequant grouped GEMM; and the combine
 * y[t] = sum_j w[t,j] O[inv_perm[t*k+j]] (fixed order over j) -> y [T, H].
 * x [T, H] bf16; wgu_codes [E, 2I, H/2], wgu_scales fp16 [E, 2I, H/g];
 * wd_codes [E, H, I/2], wd_scales fp16 [E, H, I/g] (OFT_W_BF16: bf16
 * weights in the code arrays, see oft_moe_desc); R_ops [E, 2I/b, 2, b, b]. */
int32_t oft_moe_grouped_fwd(const oft_moe_desc* d, const uint16_t* x, const float* logits,
                            const uint8_t* wgu_codes, const uint16_t* wgu_scales,
                            const uint8_t* wd_codes, const uint16_t* wd_scales,
                            const uint16_t* R_ops, const oft_moe_routing* rt,
                            uint16_t* h_saved, uint16_t* y, void* ws, size_t ws_bytes,
                            void* stream);

/* Reference-policy forward of the MoE layer: the frozen base alone, every
 * expert's gate/up projection without its adapter rotation (the pages'
 * section "Five design features of the adapter-first architecture" takes the
 * KL reference from the frozen base, so no copy of the actor is kept).  The
 * same routing, grouped dequant GEMMs, SwiGLU, down projection and combine
 * as oft_moe_grouped_fwd, with the rotation epilogue left out: y is
 * bit-identical to oft_moe_grouped_fwd's with Q = 0 (R exactly I).
 * h_or_null, when set, receives the un-rotated gate/up output [P, 2I] in
 * permuted order (nothing reads it back: a reference pass has no backward).
 * Arguments otherwise as oft_moe_grouped_fwd, without R_ops; the block size
 * b is validated but plays no part.  Errors as oft_moe_grouped_fwd. */
int32_t oft_moe_grouped_fwd_base(const oft_moe_desc* d, const uint16_t* x, const float* logits,
                                 const uint8_t* wgu_codes, const uint16_t* wgu_scales, const uint8_t* wd_codes,
                                 const uint16_t* wd_scales, const oft_moe_routing* rt, uint16_t* h_or_null,
                                 uint16_t* y, void* ws, size_t ws_bytes, void* stream);

/* Backward of <dy, y> with the routing fixed: dx [T, H] bf16 through the
 * experts, dq fp32 [E, 2I/b, b(b-1)/2] (zero for inactive experts) and
 * dw fp32 [T, k] = <dy[t], W_d,e . act>.  Any of the three may be NULL.
 * Reads rt and h_saved from the forward; re-dequantises the weights. */
int32_t oft_moe_grouped_bwd(const oft_moe_desc* d, const uint16_t* dy, const oft_moe_routing* rt,
                            const uint16_t* h_saved, const uint8_t* wgu_codes,
                            const uint16_t* wgu_scales, const uint8_t* wd_codes,
                            const uint16_t* wd_scales, const float* R_f32,
                            const uint16_t* R_ops, uint16_t* dx_or_null, float* dq_or_null,
                            float* dw_or_null, void* ws, size_t ws_bytes, void* stream);

/* Router backward: d_logits fp32 [T, E] from dw fp32 [T, k] (the gradient of
 * the combine weights, as oft_moe_grouped_bwd writes it) through the softmax
 * of the router-selected experts (the pages' section "Dedicated optimisation
 * for low-precision MoE models" routes every token to the experts its router
 * selects).  The selection topk_idx [T, k] (int32, from oft_moe_route) is
 * held fixed: top-k is piecewise constant in the logits.  renorm = 0:
 * dl_e = p_e (g_e - S) for every expert, p the softmax of the row, g_e the
 * dw of e if selected (else 0), S = sum_j dw_j w_j; renorm = 1: the selected
 * experts get w_m (dw_m - S), the others 0.  p and w are recomputed from
 * logits [T, E] exactly as oft_moe_route computes them; a NaN logit gets no
 * gradient and an index outside [0, E) selects nothing.  Errors: as oft_moe_route (descriptor), OFT_EINVAL (a NULL or
 * misaligned pointer when T > 0).  T == 0 is a no-op. */
int32_t oft_moe_router_bwd(const oft_moe_desc* d, const float* logits, const int32_t* topk_idx,
                           const float* dw, float* d_logits, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* OFT_H_ */
