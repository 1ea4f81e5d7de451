/*
 * rs.h - C ABI of the ReplaySSM SSM-layer decode step on AMD Instinct MI355X (gfx950).
 *
 * What the library computes (ReplaySSM news coverage, sitech.ge page, section
 * "How ReplaySSM works"): each sequence's SSM-layer state is kept as a
 * high-precision checkpoint plus a buffer (ring) of the most recent input
 * records. A non-flush step appends the current input and computes the output
 * from checkpoint + buffer without writing any state. When the 16-entry buffer
 * fills, a flush step folds the buffered inputs into the checkpoint, writes it
 * once and clears the buffer. Outputs equal those of conventional decoding up
 * to floating-point rounding. Speculative decoding appends draft inputs and
 * commits the accepted prefix by moving a pointer, with no state snapshots
 * (same page, "Reducing state traffic and simplifying rollback"). An optional
 * low-precision copy of the checkpoint serves reads while the recurrence keeps
 * its own precision (same page, "Bounding quantization error").
 *
 * Layer types (news.hamidun.com ReplaySSM page, "Why hybrid models became the
 * norm"): Mamba-2 and Gated DeltaNet.
 *
 *   Mamba-2, per sequence b and head h (group g = h / (nheads / ngroups)):
 *     a = exp(dt * A[h]);  H = a*H + dt * x B^T;  y = H C + D[h] * x
 *   Gated DeltaNet, per sequence b and value head h (qk head = h / (n_v / n_qk)):
 *     alpha = exp(g);  S = alpha * S (I - beta k k^T) + beta v k^T;  o = S q
 *
 * ---------------------------------------------------------------------------
 * Conventions shared by every entry point
 * ---------------------------------------------------------------------------
 * Ownership. The caller allocates and owns every device buffer, sized from
 *   the rs_layer that rs_init fills. The library allocates nothing and never
 *   synchronises; there is nothing to destroy. Its only global state is the
 *   static device array of rs_spec_commit_static (one per device).
 * Pointers. Device pointers (hipMalloc'd or equivalent), 16-byte aligned.
 *   rs_layer, rs_buffers, rs_inputs and rs_params structs themselves are host
 *   memory, read during the call only.
 * Streams. `stream` is a hipStream_t (NULL = the default stream). Every kernel
 *   is enqueued on it and the call returns without waiting. Calls that touch
 *   the same buffers must be ordered on one stream by the caller. Calls that
 *   overlap on the same buffers race.
 * Errors. Problems visible on the host return a negative rs_status and launch
 *   nothing. Contract violations that depend on device-resident buffer state
 *   (see rs_meta.err) set sticky bits in that sequence's meta record and leave
 *   the sequence's checkpoint, buffer and counters unchanged; its outputs for
 *   that call are not written.
 * Initial state. The caller zero-fills `meta` (and `ring`, optionally),
 *   writes the initial checkpoint in the layout below, and, if a read copy is
 *   configured, calls rs_requant_read_copy once before the first step.
 *
 * ---------------------------------------------------------------------------
 * Device layouts (all row-major, innermost index last)
 * ---------------------------------------------------------------------------
 * Mamba-2 (P = headdim, N = dstate, G = ngroups, R = ring = 16):
 *   checkpoint  RS_F32: float [batch][nheads][N][P]; element H[b][h][p][n] is
 *               at ((b*nheads + h)*N + n)*P + p (the state stored transposed,
 *               headdim innermost).
 *               RS_F16: binary16 in the same order.
 *               RS_FP8E4M3: uint8 E4M3FN codes in the same order, then
 *               float scale[batch][nheads] at byte offset ck_scale_off.
 *               RS_NVFP4: an NVFP4 block (below) per matrix.
 *   ring        in_dtype arrays at the byte offsets in rs_layer:
 *               x [batch][nheads][R][P], B [batch][G][R][N], C [batch][G][R][N],
 *               dt [batch][nheads][R]. Buffer entry i of sequence b (0-based,
 *               i < len + nd) is in slot (n_ckpt + i) mod R.
 *   inputs      x [batch][nheads][P], B and C [batch][G][N], dt [batch][nheads]
 *               (in_dtype); drafts stack K tokens in front: [K][batch][...].
 *   params      A, D: float [nheads].
 *   output      y: float [batch][nheads][P]; for drafts [K][batch][nheads][P].
 * Gated DeltaNet (dk = head_k_dim, dv = head_v_dim, Hv = n_v_heads, Hk = n_qk_heads):
 *   checkpoint  RS_F32: float [batch][Hv][dk][dv]; element S[b][h][v][k] is at
 *               ((b*Hv + h)*dk + k)*dv + v.
 *   ring        q and k [batch][Hk][R][dk] (in_dtype), v [batch][Hv][R][dv]
 *               (in_dtype), g and beta float [batch][Hv][R]; and, beside each
 *               held entry i, u float [batch][Hv][R][dv]: its row of the
 *               triangular system u_i = beta_i (v_i - alpha_i S_{i-1} k_i),
 *               which depends only on the checkpoint and entries <= i, so the
 *               library writes it once, on the step that appends entry i.
 *   inputs      q, k [batch][Hk][dk], v [batch][Hv][dv] (in_dtype);
 *               g (= log alpha) and beta: float [batch][Hv]; drafts stack K
 *               tokens in front: [K][batch][...].
 *   output      o: float [batch][Hv][dv]; for drafts [K][batch][Hv][dv].
 * Kimi Delta Attention (RS_KDA; Kimi Linear, Moonshot AI 2025; named as an SSM
 *   layer type on the news.hamidun.com ReplaySSM page, "Why hybrid models
 *   became the norm"): S_t = S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T)
 *   + beta_t v_t k_t^T, o_t = S_t q_t, with alpha_t = exp(g_t) a vector over
 *   the dk key channels. Everything as for Gated DeltaNet except g: float
 *   [batch][Hv][dk] per token (drafts [K][batch][Hv][dk]), and the ring's g
 *   float [batch][Hv][R][dk]. The speculative calls work as for Gated
 *   DeltaNet (the draft records are verified inside the KDA layer).
 * NVFP4 block (read copy, or the uniform NVFP4 checkpoint), for the stored
 *   matrices M[b][h] of rows x cols (rows = N or dk, cols = P or dv):
 *     codes   uint8 [batch][heads][rows][cols/2]: two E2M1 codes per byte,
 *             even column in the low nibble; code = sign<<3 | magnitude index
 *             into {0, .5, 1, 1.5, 2, 3, 4, 6};
 *     scales  uint8 [batch][heads][rows][cols/16] E4M3FN block scales, at
 *             byte offset nv_scale_off;
 *     tscale  float [batch][heads] tensor scales, at byte offset nv_tscale_off.
 *   Value = e2m1(code) * (e4m3(scale) * tscale). Quantization, in float32:
 *   tscale = amax/2688 (1 if 0); scale = E4M3(block_amax / (6*tscale)),
 *   round-to-nearest-even, saturating; code = E2M1(x / (e4m3(scale)*tscale)),
 *   round-to-nearest-even, saturating (all zero if that divisor is 0).
 * Snapshots (conventional mode with max_draft > 0): float
 *   [max_draft][batch][heads][rows][cols], the state after each draft.
 * meta: rs_meta[batch], followed by library work space (meta_bytes in all).
 */
#ifndef RS_H
#define RS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t rs_status;

/* status codes */
#define RS_OK 0
#define RS_E_ARG (-1)        /* null pointer, bad size, inconsistent shape */
#define RS_E_DTYPE (-2)      /* unsupported dtype or dtype combination */
#define RS_E_ALIGN (-3)      /* device pointer not 16-byte aligned */
#define RS_E_MODE (-4)       /* call not valid for the layer's mode or config */
#define RS_E_LAUNCH (-5)     /* a kernel launch failed (hipGetLastError) */
#define RS_E_UNSUPPORTED (-6)/* shape outside the compiled kernel set */

/* layer kinds */
#define RS_MAMBA2 1
#define RS_GDN 2
#define RS_KDA 3   /* Kimi Delta Attention: the Gated DeltaNet layout, gate per key channel */

/* modes */
#define RS_REPLAY 0          /* checkpoint + ring (ReplaySSM) */
#define RS_CONVENTIONAL 1    /* live state read and written every step (baseline) */

/* dtypes */
#define RS_NONE 0
#define RS_F32 1
#define RS_BF16 2
#define RS_F16 3
#define RS_FP8E4M3 4
#define RS_NVFP4 5

/* sticky device-side error bits in rs_meta.err */
#define RS_ERR_FULL 1        /* non-flush step on a full buffer (len == ring-1) */
#define RS_ERR_OVERFLOW 2    /* append would exceed the ring, or K out of range */
#define RS_ERR_COMMIT 4      /* commit count outside [0, nd] */
#define RS_ERR_PENDING 8     /* plain step while drafts are pending */

typedef struct rs_config {
  int32_t kind;          /* RS_MAMBA2 | RS_GDN | RS_KDA */
  int32_t mode;          /* RS_REPLAY | RS_CONVENTIONAL */
  int32_t batch;         /* sequences, >= 1 */
  int32_t nheads, headdim, dstate, ngroups;              /* Mamba-2 */
  int32_t n_qk_heads, n_v_heads, head_k_dim, head_v_dim; /* Gated DeltaNet */
  int32_t ring;          /* buffer entries; must be 16 */
  int32_t max_draft;     /* 0 = no speculative decoding; else 1..ring/2 */
  int32_t in_dtype;      /* RS_F32 | RS_BF16 (GDN g and beta are always float) */
  int32_t ckpt_dtype;    /* RS_F32 | RS_F16 | RS_FP8E4M3 | RS_NVFP4 (uniform comparator);
                            Gated DeltaNet and KDA: RS_F32, or RS_F16 / RS_FP8E4M3 in
                            replay mode without a read copy on 16 x 16 and 128 x 128
                            states (RS_E_UNSUPPORTED on 64 x 64) */
  int32_t read_copy;     /* RS_NONE | RS_NVFP4 (replay mode). Gated DeltaNet and KDA:
                            with an RS_F32 checkpoint; the flush and the commit fold
                            rewrite the copy of the states they fold in the same launch;
                            rs_step rewrites it in a second launch on the same stream
                            (its flushes fold in column slices); whatever fuse_requant
                            says */
  int32_t fuse_requant;  /* Mamba-2: 1: flush and commit-fold rewrite the read copy in
                            their epilogue; 0: the caller calls rs_requant_read_copy */
} rs_config;

/* Per-sequence buffer counters (32 bytes). */
typedef struct rs_meta {
  int64_t n_ckpt;        /* tokens folded into the checkpoint */
  int32_t len;           /* committed buffer entries */
  int32_t nd;            /* pending draft entries */
  int32_t err;           /* sticky RS_ERR_* bits */
  uint32_t arrive;       /* workgroups counted in during a step launch; zero between calls */
  int32_t reserved[2];
} rs_meta;

/* Filled by rs_init. Plain data; the caller keeps it. */
typedef struct rs_layer {
  rs_config cfg;
  int32_t heads;         /* state matrices per sequence: nheads | n_v_heads */
  int32_t in_heads;      /* B/C groups | qk heads */
  int32_t rows, cols;    /* stored matrix: rows = dstate | dk, cols = headdim | dv */
  uint64_t ckpt_bytes, ring_bytes, read_copy_bytes, meta_bytes, snap_bytes;
  /* ring arrays, byte offsets into the ring buffer */
  uint64_t ring_x_off, ring_B_off, ring_C_off, ring_dt_off;               /* Mamba-2 */
  uint64_t ring_q_off, ring_k_off, ring_v_off, ring_g_off, ring_beta_off; /* GDN */
  uint64_t ring_u_off;   /* GDN: solution row u of each held entry (library-maintained) */
  /* checkpoint extras, byte offsets into the checkpoint buffer */
  uint64_t ck_scale_off;                     /* RS_FP8E4M3 per-matrix scales */
  uint64_t ck_nv_scale_off, ck_nv_tscale_off;/* RS_NVFP4 checkpoint */
  /* read copy, byte offsets into the read-copy buffer */
  uint64_t nv_scale_off, nv_tscale_off;
  uint64_t meta_work_off;                    /* library work space inside meta */
  uint32_t magic;                            /* set by rs_init */
  uint32_t reserved;
} rs_layer;

typedef struct rs_buffers {
  void* ckpt;            /* checkpoint (or live state in conventional mode) */
  void* ring;            /* replay mode */
  void* read_copy;       /* when read_copy != RS_NONE */
  void* meta;            /* replay mode: meta_bytes, zero-filled before first use */
  void* snap;            /* conventional mode with max_draft > 0 */
} rs_buffers;

typedef struct rs_inputs {
  const void *x, *B, *C, *dt;          /* Mamba-2 */
  const void *q, *k, *v, *g, *beta;    /* Gated DeltaNet */
} rs_inputs;

typedef struct rs_params {
  const float *A, *D;    /* Mamba-2 per-head; unused for GDN */
} rs_params;

/* Validate cfg and fill *out with sizes and offsets. Host only: no device
 * call, no allocation. Returns RS_E_ARG / RS_E_DTYPE / RS_E_MODE /
 * RS_E_UNSUPPORTED for an invalid or uncompiled configuration. */
rs_status rs_init(const rs_config* cfg, rs_layer* out);

/* Conventional decode step (sitech.ge ReplaySSM page, "How ReplaySSM works":
 * conventional decoding reads and writes the full state at every step).
 * Conventional-mode layers only; y receives the step output. */
rs_status rs_step_conventional(const rs_layer* L, const rs_buffers* buf, const rs_inputs* in,
                               const rs_params* prm, float* y, void* stream);

/* Non-flush step (same page and section): appends the current input to
 * buffer slot (n_ckpt + len) mod 16, writes y from checkpoint (or its read
 * copy) plus buffer, writes no state; len += 1. Replay mode. Device errors:
 * RS_ERR_FULL if len == 15, RS_ERR_PENDING if drafts are pending. */
rs_status rs_step_nonflush(const rs_layer* L, const rs_buffers* buf, const rs_inputs* in,
                           const rs_params* prm, float* y, void* stream);

/* Flush step (same page and section): folds the len stored entries and the
 * current input into the checkpoint, writes it once (and the read copy when
 * fuse_requant), writes y; n_ckpt += len + 1, len = 0. Valid at any fill.
 * Replay mode. Device error: RS_ERR_PENDING. */
rs_status rs_step_flush(const rs_layer* L, const rs_buffers* buf, const rs_inputs* in,
                        const rs_params* prm, float* y, void* stream);

/* Self-scheduling step (continuous batching; the flush rule of sitech.ge,
 * "How ReplaySSM works", applied per sequence): in one launch, a sequence
 * whose buffer is full (len == 15) takes the flush step and every other
 * sequence the non-flush step, so sequences at different fills share a batch
 * and a lockstep batch's flush work is spread over steps once fills differ.
 * Same arguments, outputs and device errors as the two calls above. Replay
 * mode. */
rs_status rs_step(const rs_layer* L, const rs_buffers* buf, const rs_inputs* in,
                  const rs_params* prm, float* y, void* stream);

/* Reuse sequence slots (continuous batching): clears the counters of the
 * listed sequences (n_ckpt = len = nd = 0, error bits cleared), so each starts
 * with an empty buffer; the sequences' checkpoint rows then hold whatever the
 * caller writes there as the new initial state (call rs_requant_read_copy
 * afterwards if a read copy is configured). seqs: device int32[count]; entries
 * outside [0, batch) are skipped; count == 0 launches nothing. Replay mode. */
rs_status rs_reset_slots(const rs_layer* L, const rs_buffers* buf, const int32_t* seqs, int32_t count,
                         void* stream);

/* Copy whole sequence states (prefix caching, forks). The state of a sequence
 * at any token is its checkpoint, its buffer entries and its counters, with no
 * per-token snapshot (sitech.ge ReplaySSM page, "Reducing state traffic and
 * simplifying rollback"), so saving it, restoring it or forking it is a copy
 * of those regions: for i < count, the state of sequence src_seqs[i] of `src`
 * (layer Ls) replaces that of sequence dst_seqs[i] of `dst` (layer Ld) —
 * checkpoint rows with their scales, read copy, all 16 ring slots of every
 * ring array (GDN / KDA solved rows u included), and the counters n_ckpt, len,
 * nd, err (the arrival count stays). A restored sequence continues exactly as
 * the saved one would have: same outputs, same flush schedule. Ls and Ld must
 * have identical configurations except batch (src and dst may be the same
 * buffers of one layer, e.g. a cache of B_cache sequences beside a decode
 * batch); pairs with an index outside its layer's batch are skipped.
 * src_seqs, dst_seqs: device int32[count], count <= 65535. Destinations must
 * be distinct and must not be sources of the same call (those copies would
 * race). Conventional mode copies the checkpoint (live state) only. */
rs_status rs_copy_slots(const rs_layer* Ls, const rs_buffers* src, const int32_t* src_seqs,
                        const rs_layer* Ld, const rs_buffers* dst, const int32_t* dst_seqs,
                        int32_t count, void* stream);

/* Mamba-2 block around the SSM step (Dao and Gu 2024; the ReplaySSM pages name
 * the layer type only). Both calls take a Mamba-2 layer; K = 1 for a plain
 * token, or the K drafts of a speculative round (K <= max_draft).
 *
 * Short causal convolution (depthwise, width W <= 4, bias, then SiLU) over the
 * channels xBC = [x | B | C], C_ch = nheads*headdim + 2*ngroups*dstate:
 *   out_t[c] = silu(bias[c] + sum_{k<W} weight[c][k] * xBC_{t-W+1+k}[c]).
 * Its state, the last W-1 inputs, is a ring of recent inputs like the SSM
 * buffer (sitech.ge ReplaySSM page, "Reducing state traffic and simplifying
 * rollback"): conv_ring, in_dtype [batch][16][C_ch] (batch * 16 * C_ch *
 * sizeof(in) bytes, caller-owned), holds the input of token position q in
 * slot q mod 16, where the next position of sequence b is n_ckpt + len of the
 * layer's meta (replay mode). Call it before the SSM call of the same tokens:
 * it reads positions p-W+1..p-1, writes the K inputs at p..p+K-1 and the
 * outputs x [K][batch][nheads][headdim], B and C [K][batch][ngroups][dstate]
 * (in_dtype; bf16 rounded to nearest even), ready for the SSM call. A
 * speculative commit needs nothing here (the SSM commit advances the
 * position; slots of rejected drafts are overwritten later). A new sequence's
 * caller writes its last W-1 prompt inputs, or zeros, at positions -W+1..-1
 * (slots 16-W+1..15 when n_ckpt = len = 0); rs_copy_slots does not copy this
 * buffer (copy the sequence's [16][C_ch] row with it). Sequences with drafts
 * pending or without room for K entries (len + K > 16) are skipped, outputs
 * untouched, as the SSM call refuses them. xbc: in_dtype [K][batch][C_ch];
 * weight float [C_ch][W]; bias float [C_ch] or NULL. d_inner and
 * ngroups*dstate must be multiples of 8; pointers (bias included) 16-byte
 * aligned. */
rs_status rs_conv_step(const rs_layer* L, const rs_buffers* buf, void* conv_ring, const void* xbc,
                       int32_t K, const float* weight, const float* bias, int32_t width,
                       void* x, void* B, void* C, void* stream);

/* Gated RMS norm of the SSM output (same block; gate applied before the norm):
 *   v = y * silu(z);  out = v / sqrt(mean_group(v^2) + eps) * weight
 * over norm_groups groups of d_inner / norm_groups consecutive channels of
 * the flattened y [nheads*headdim]. y float [K][batch][d_inner] (the SSM
 * call's output), z and out in_dtype [K][batch][d_inner] (bf16 rounded to
 * nearest even), weight float [d_inner]; pointers 16-byte aligned, group size
 * a multiple of 4 (RS_E_UNSUPPORTED otherwise). Either mode. */
rs_status rs_gated_norm(const rs_layer* L, int32_t K, const float* y, const void* z,
                        const float* weight, int32_t norm_groups, float eps, void* out,
                        void* stream);

/* Speculative append (same page, "Reducing state traffic and simplifying
 * rollback": draft inputs enter the buffer until verification; verification
 * reads outputs only, as a small matrix product, without forming
 * intermediate states). `drafts` holds K stacked tokens; y receives the K
 * verify outputs [K][batch][...]. Replay mode: writes the drafts to the
 * slots after the committed entries, nd = K, no state write (device error
 * RS_ERR_OVERFLOW when nd != 0 or len + K > 16). Conventional mode: the
 * snapshot baseline; steps the live state through the drafts and writes the
 * state after each draft to snap[d]. Every layer kind (for the delta rules
 * prm may be NULL; each draft's solved row u is written beside it in the
 * ring, and it stays valid for an accepted prefix because it depends only on
 * the checkpoint and earlier entries); 1 <= K <= max_draft. */
rs_status rs_spec_append(const rs_layer* L, const rs_buffers* buf, const rs_inputs* drafts,
                         int32_t K, const rs_params* prm, float* y, void* stream);

/* Speculative commit (same section): accepted is a device int32[batch].
 * Replay mode: len += accepted[b], nd = 0; rejected drafts are dropped by
 * the pointer move alone. If then len > 16 - max_draft, the len committed
 * entries are folded into the checkpoint (one write), n_ckpt += len, len = 0.
 * Device error RS_ERR_COMMIT when accepted[b] is outside [0, nd].
 * Conventional mode: live state = snap[accepted[b] - 1] where accepted[b] >= 1
 * (values outside [0, max_draft] leave the sequence unchanged). Every layer
 * kind; prm (A, D) is required for Mamba-2 only. */
rs_status rs_spec_commit(const rs_layer* L, const rs_buffers* buf, const int32_t* accepted,
                         const rs_params* prm, void* stream);

/* rs_spec_commit for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops that forbid allocation): identical
 * arguments, results and errors, but the commit's fold list (the ordered list
 * of sequences whose committed entries are folded, and its count) lives in a
 * static device array inside the library instead of the meta buffer's work
 * space. Nothing is allocated, here or at set-up; the array (128 KiB per
 * device, held until the process ends) is resolved on the first call on each
 * device. Limit: batch <= 8192 (RS_E_ARG beyond it). Every call on one device
 * shares that array: calls that overlap on one device, from any stream or
 * layer, race; order them. RS_E_LAUNCH if the runtime cannot give the
 * array's address. */
rs_status rs_spec_commit_static(const rs_layer* L, const rs_buffers* buf, const int32_t* accepted,
                                const rs_params* prm, void* stream);

/* Rewrite the whole NVFP4 read copy from the stored checkpoint (same page,
 * "Bounding quantization error"). Needs read_copy == RS_NVFP4. Bit-identical
 * to what a flush with fuse_requant writes for the same checkpoint. */
rs_status rs_requant_read_copy(const rs_layer* L, const rs_buffers* buf, void* stream);

/* Static string for a status code. */
const char* rs_status_string(rs_status s);

/* Library version, major*10000 + minor*100 + patch. */
int32_t rs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RS_H */
