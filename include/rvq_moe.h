/*
 * rvq_moe.h -- C ABI of the routed RVQ-MoE decode layer for MI355X (gfx950).
 *
 * One Mixture-of-Experts layer whose expert weights are stored as 3-stage
 * residual vector quantisation: three 256-entry codebooks over 8-wide weight
 * vectors, one code byte per stage, 3.00 bits per weight.  The layer routes
 * every token to its top-k experts and evaluates each expert's SwiGLU FFN
 * (gate, up, down) straight from the codes through tables of partial dot
 * products built in LDS, never materialising a dense matrix.
 *
 * Sources:
 *   [FR] "Exécuter Kimi K3 avec 29 Go de RAM à 0,50 tok/s" (fr.news.hada.io,
 *        topic 32035):
 *        - "Quantification et exactitude": the RVQ format (3 stages, 256
 *          entries, 8-dim vectors, 3.00 bits/weight) and its evaluation (a
 *          table of partial dot products, 3 lookups and 2 additions per row).
 *        - "Architecture de streaming depuis le disque": gate, up and down of
 *          one expert are contiguous so one expert is one read; every record
 *          read is checked (magic, expert id, offset range) and, on request,
 *          its payload's crc32.
 *        - "Lecture anticipée et prédiction du routeur": the router of a layer
 *          decides 16 expert ids and expert reads are consumed as they land.
 *        - "Objectif et forme d'implémentation de WASTE": a small public C API
 *          (open, set a memory limit, run, close) called from Python by ctypes.
 *        - "Budget RAM et fenêtre de performance étroite": 16 experts per token
 *          per layer; the engine refuses to start below its minimum budget.
 *   [RU] "WASTE: запускаем полную Kimi K3 на MacBook Pro с 64 ГБ памяти"
 *        (feed.hirify.me), "Расчёт строится на устройстве MoE": 16 experts per
 *        layer, gate/up/down stored back to back, the matrix never unfolded.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers (HIP, the device current at rvq_moe_open)
 *     unless stated otherwise.  Arrays are dense, row-major, little-endian.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously on it; nothing in route_topk or
 *     layer_forward synchronises the host.
 *   - Return value: RVQ_MOE_OK (0) or a negative rvq_moe_status.  Arguments
 *     are validated before anything is enqueued; on error nothing is
 *     enqueued, nothing is allocated and no output is written.
 *     rvq_moe_last_error() gives a human-readable reason.
 *   - A handle is not thread-safe (its workspace is shared by its calls);
 *     distinct handles hold no shared state.  Calls that overlap on one handle
 *     from different streams race.
 *   - Residency: the kernels of rvq_moe_layer_forward (table path),
 *     rvq_moe_route_forward and rvq_moe_route_topk with one token are
 *     persistent grids whose workgroups wait for one another, so each assumes
 *     the whole GPU is free for its grid.  Such calls, of any handles, must not
 *     run concurrently on different streams: order them (same stream, or
 *     events).  Otherwise two partly resident grids can wait on each other
 *     until the bounded inter-workgroup wait (~0.5 s) gives up, and the calls
 *     fail with RVQ_MOE_EDEVICE (timeout flag) at the next sync; the device
 *     never hangs.  Copies (the slot cache) and the router of a streaming
 *     handle (codes_location PINNED_*, which always takes the router kernels
 *     that need no co-resident grid) may overlap them freely, e.g. router
 *     lookahead on a side stream (rvq_moe_prefetch).
 */
#ifndef RVQ_MOE_H
#define RVQ_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RVQ_MOE_ABI_VERSION 6

typedef enum rvq_moe_status {
    RVQ_MOE_OK = 0,
    RVQ_MOE_EINVAL = -1,   /* bad dimension, pointer, token count or id */
    RVQ_MOE_ENOTSUP = -2,  /* valid but unsupported format (stages != 3, codes != 256, vec != 8, ...) */
    RVQ_MOE_EBUDGET = -3,  /* slot cache smaller than one token's working set (0 < cache_slots < top_k) */
    RVQ_MOE_ENOMEM = -4,   /* device or pinned allocation failed */
    RVQ_MOE_EHIP = -5,     /* a HIP runtime call or launch failed */
    RVQ_MOE_EDEVICE = -6,  /* deferred: a kernel saw an expert id outside [0, n_experts) */
    RVQ_MOE_ECORRUPT = -7  /* an expert record failed its integrity check (see rvq_moe_record_trailer) */
} rvq_moe_status;

/* Default chunk-path threshold (tokens per layer_forward call): where the
 * chunk path (with the default adaptive dispatch below) overtakes the table
 * path for d=7168, ffn=2048, E=384, top-16 on one MI355X (32 tokens: table
 * 1.53 ms, chunk 1.61 ms; 48 tokens: table 2.35 ms, chunk 2.23 ms; 64 tokens:
 * table 3.08 ms, chunk 2.73 ms).  Other shapes may set their own. */
#define RVQ_MOE_CHUNK_MIN_TOKENS 40

/* Default of lut_expert_tokens (see rvq_moe_desc): the best of 3..6 measured
 * at that shape (96 tokens per call: 4.05 ms against 4.97 ms with every expert
 * on the matrix cores). */
#define RVQ_MOE_LUT_EXPERT_TOKENS 4

typedef enum rvq_moe_cb_dtype {
    RVQ_MOE_CB_F32 = 0,    /* IEEE binary32 codebook entries */
    RVQ_MOE_CB_F16 = 1     /* IEEE binary16 codebook entries */
} rvq_moe_cb_dtype;

typedef enum rvq_moe_codes_location {
    RVQ_MOE_CODES_DEVICE = 0,       /* canonical codes in device memory; copied and repacked at open */
    RVQ_MOE_CODES_PINNED_HOST = 1,  /* canonical codes in pinned host memory; open writes the handle's own
                                       pinned bank from them (see rvq_moe_write_bank) */
    RVQ_MOE_CODES_PINNED_BANK = 2   /* `codes` is a bank written by rvq_moe_write_bank, in pinned host
                                       memory; borrowed (it must outlive the handle) */
} rvq_moe_codes_location;

/*
 * Expert-record bank of a streaming handle.  [FR] "Architecture de streaming
 * depuis le disque": an expert's gate, up and down form one record read in
 * one piece; each record read is checked for its magic, its expert id and its
 * offset range, so that a truncated or wrongly assembled bank cannot hand out
 * another expert's weights; a crc32 of the payload is checked only on request
 * (about 1 % of the time on K3 there); codebooks carry no checksum.
 *
 * Record e of a bank occupies bytes [e * stride, (e + 1) * stride)
 * (rvq_moe_bank_layout gives stride and payload_bytes; stride is a multiple of
 * 4096): the payload (the expert's codes in the library's internal layout),
 * zeros up to the next 4096-byte boundary, then a 4096-byte trailer page
 * holding an rvq_moe_record_trailer followed by zeros.  Every copy of a record
 * into an HBM slot is followed, on the device and before any kernel reads the
 * slot, by the trailer checks (magic and version; expert == e and n_experts;
 * offset == e * stride, payload_bytes, d and ffn) and, with verify_records,
 * by the CRC-32 of the payload as it landed in HBM.  A failure is reported
 * as RVQ_MOE_ECORRUPT by every later rvq_moe_sync and by rvq_moe_close (it is
 * not cleared: the bank is damaged); outputs of calls that read the record
 * are unspecified.  Open checks every trailer of a PINNED_BANK on the host.
 * CRC-32 here is the one of zlib and IEEE 802.3 (reflected polynomial
 * 0xEDB88320, initial value and final xor 0xFFFFFFFF; "123456789" -> 0xCBF43926).
 */
#define RVQ_MOE_RECORD_MAGIC 0x52515652u /* the bytes "RVQR" */
#define RVQ_MOE_RECORD_VERSION 1u
typedef struct rvq_moe_record_trailer {
    uint32_t magic;          /* RVQ_MOE_RECORD_MAGIC */
    uint32_t version;        /* RVQ_MOE_RECORD_VERSION */
    uint32_t expert;         /* the expert whose codes the payload holds */
    uint32_t n_experts;      /* E of the bank */
    uint64_t offset;         /* byte offset of this record in the bank (expert * stride) */
    uint64_t payload_bytes;  /* payload size */
    int32_t d, ffn;          /* layer shape the payload is laid out for */
    uint32_t crc32;          /* CRC-32 of the payload_bytes payload bytes */
    uint32_t reserved;       /* 0 */
} rvq_moe_record_trailer;
/* Flags of a failed record check (rvq_moe_last_error names them and the expert). */
#define RVQ_MOE_RECORD_BAD_MAGIC 1 /* magic or version */
#define RVQ_MOE_RECORD_BAD_ID 2    /* expert or n_experts */
#define RVQ_MOE_RECORD_BAD_RANGE 4 /* offset, payload_bytes, d or ffn */
#define RVQ_MOE_RECORD_BAD_CRC 8   /* payload CRC-32 (checked only with verify_records) */

/*
 * Layer description, read only during rvq_moe_open.
 *
 *   d, ffn       hidden size and expert FFN width; both multiples of 8 (the
 *                vector width), d <= 65536, ffn <= 65536.
 *   n_experts    E, 1 <= E <= 1024.     top_k   k, 1 <= k <= min(E, 64).
 *   n_stages, n_codes, vec_dim   must be 3, 256, 8 ([FR] "Quantification et
 *                exactitude"); anything else is RVQ_MOE_ENOTSUP.
 *   codebook_dtype  rvq_moe_cb_dtype.
 *   router_w     fp32 [d][E] router matrix: logits[e] = sum_i x_i W[i][e].
 *   codebooks    [E][3 matrices: gate, up, down][3 stages][256][8] entries of
 *                codebook_dtype.  A weight is c1 + c2 + c3, the sum of its
 *                three stage vectors' entries; no scale, no bias.  Any finite
 *                values: fp32 codebooks are scaled per (expert, matrix) by an
 *                exact power of two inside the table build, so the ~1e-6
 *                relative accuracy of the table path holds at every scale
 *                (fp32 range); non-finite entries propagate to the outputs.
 *   codes        [E][record] with record = gate [ffn][d/8][3] u8, then up
 *                [ffn][d/8][3] u8, then down [d][ffn/8][3] u8: byte s of
 *                (row, slice j) indexes stage s's codebook for the 8 weights
 *                row[8j .. 8j+7].  Record bytes = 9 * d * ffn / 8.
 *                With codes_location PINNED_BANK, `codes` is instead a bank
 *                written by rvq_moe_write_bank for the same d, ffn, E.
 *   codes_location  rvq_moe_codes_location.  PINNED_HOST and PINNED_BANK
 *                stream the codes through cache_slots HBM slots (both need
 *                cache_slots >= top_k); DEVICE keeps them all resident
 *                (cache_slots must be 0).
 *   cache_slots  0 = all experts resident.  Otherwise the number of HBM expert
 *                slots; must be >= top_k (RVQ_MOE_EBUDGET), mirroring the
 *                refusal to start below one token's working set.
 *   pre_rmsnorm  nonzero: x_hat = x / sqrt(mean(x^2) + eps) feeds both the
 *                router and the experts (unit norm weight).  eps is double.
 *   residual     nonzero: layer_forward returns x + MoE(x_hat) instead of
 *                MoE(x_hat).
 *   max_tokens   largest n_tokens any later call will pass (sizes the
 *                per-handle workspace, allocated once at open).
 *   chunk_min_tokens  layer_forward calls with n_tokens >= this take the chunk
 *                path (tokens grouped by expert, weights rebuilt as bf16 and
 *                contracted on the matrix cores, see rvq_moe_layer_forward);
 *                0 = the library default (RVQ_MOE_CHUNK_MIN_TOKENS); a value
 *                above max_tokens never takes it (and allocates nothing for
 *                it).  Must be >= 0.
 *   lut_expert_tokens  adaptive dispatch inside a chunk-path call: an expert
 *                routed fewer tokens than this is evaluated by the table path
 *                (fp32, per-token tables) instead of the matrix cores, as long
 *                as the pairs so handed over fit the table path's order table
 *                (512 pairs; experts in id order).  0 = the library default
 *                (RVQ_MOE_LUT_EXPERT_TOKENS); 1 = every expert on the matrix
 *                cores.  Streaming handles always use 1.  Must be >= 0.
 *   verify_records  streaming handles: nonzero = also check the CRC-32 of
 *                every record copied into a slot (see rvq_moe_record_trailer);
 *                the trailer checks always run.  Ignored for DEVICE codes.
 *   deterministic  0 or 1.  1: every output is a fixed-order sum, so repeated
 *                calls, streaming and resident codes, grouped and per-token
 *                calls and prefetching on or off all give bitwise identical
 *                y (the same tokens, ids and gates in, the same bits out).
 *                [FR] "Lecture anticipée et prédiction du routeur": reading
 *                ahead and overlapping leave the output exactly as it was.
 *                Each (token, expert) pair's output rows (per down-projection
 *                tile on the table path) go to a workspace buffer and a small
 *                kernel adds them to y in the order (expert rank, tile), after
 *                x when `residual`; gate/up partial sums are never merged
 *                across tiles; adaptive dispatch is off (lut_expert_tokens is
 *                taken as 1).  0 (the default): the layer kernels add into y
 *                with fp32 atomics, whose order varies, so outputs agree to
 *                ~1e-7 relative between runs; no extra launch and no buffer.
 *                Cost of 1 on one MI355X at d=7168, ffn=2048, E=384, top-16:
 *                +7 us per one-token routed call (+12 %), +4 % for 32-token
 *                calls, +2 % for 512-token chunk-path calls; workspace
 *                max_tokens * top_k * ceil(ffn / 256) * ceil(d / 32) * 128 bytes.
 *   stream       stream used for the upload and repack inside open.
 */
typedef struct rvq_moe_desc {
    uint32_t struct_size;       /* = sizeof(rvq_moe_desc) */
    int32_t d;
    int32_t ffn;
    int32_t n_experts;
    int32_t top_k;
    int32_t n_stages;
    int32_t n_codes;
    int32_t vec_dim;
    int32_t codebook_dtype;
    int32_t codes_location;
    int32_t cache_slots;
    int32_t pre_rmsnorm;
    int32_t residual;
    int32_t max_tokens;
    int32_t chunk_min_tokens;
    int32_t lut_expert_tokens;
    int32_t verify_records;
    int32_t deterministic;
    double eps;
    const float *router_w;
    const void *codebooks;
    const uint8_t *codes;
    void *stream;
} rvq_moe_desc;

typedef struct rvq_moe rvq_moe;

/*
 * rvq_moe_open -- validate `desc`, allocate the handle, copy the router and
 * codebooks, and repack the codes into the library's tiled internal layout.
 * [FR] "Objectif et forme d'implémentation de WASTE": the engine's C API opens
 * a model once and then runs it; [FR] "Budget RAM et fenêtre de performance
 * étroite": it refuses to start below its minimum memory budget (here
 * EBUDGET: fewer HBM slots than one token's top_k experts).
 * Synchronises `desc->stream` before returning; the caller may free every
 * input buffer afterwards (the library owns its copies and its workspace).
 * On failure *out is set to NULL and nothing stays allocated.
 * Errors: EINVAL (null desc/out/pointers, struct_size mismatch, bad dims,
 * k > E, max_tokens < 1, PINNED_* codes not in pinned host memory), ENOTSUP
 * (format), EBUDGET (0 < cache_slots < top_k), ECORRUPT (a PINNED_BANK trailer
 * fails its check: last_error names the expert), ENOMEM, EHIP.
 */
int rvq_moe_open(const rvq_moe_desc *desc, rvq_moe **out);

/*
 * rvq_moe_bank_layout -- record stride and payload size (bytes) of the bank
 * of the layer `desc` describes; the bank is n_experts * stride bytes.  Only
 * d, ffn, n_experts, top_k and the format fields of desc are read; host only.
 * Errors: EINVAL (null pointers, struct_size, bad dims), ENOTSUP (format).
 */
int rvq_moe_bank_layout(const rvq_moe_desc *desc, int64_t *record_stride, int64_t *payload_bytes);

/*
 * rvq_moe_write_bank -- write the expert-record bank of the layer `desc`
 * describes into `bank` (pinned host memory, n_experts * stride bytes, owned
 * by the caller): each record's payload (desc->codes repacked into the
 * internal layout on the device), zero fill, and its trailer with the
 * payload's CRC-32 computed on the device.  desc->codes holds canonical
 * records (as for open) in device memory (codes_location DEVICE) or pinned
 * host memory (PINNED_HOST); router_w and codebooks are not read.  Uses
 * desc->stream and synchronises it; allocates only temporary device buffers.
 * The bank can then be stored, copied, and opened as PINNED_BANK.
 * Errors: EINVAL (null pointers, bad dims, bank not pinned host memory,
 * codes_location PINNED_BANK), ENOTSUP (format), ENOMEM, EHIP.
 */
int rvq_moe_write_bank(const rvq_moe_desc *desc, uint8_t *bank);

/*
 * rvq_moe_route_topk -- router GEMV (fp64 accumulation of fp32 products),
 * then the k largest logits per token in descending order (ties to the lower
 * id) and their softmax gates (sum to 1).  [FR] "Lecture anticipée et
 * prédiction du routeur": the router decides the token's expert ids.
 *   x      [n_tokens][d] fp32 (the un-normalised input when pre_rmsnorm).
 *   ids    [n_tokens][k] int32 out.       gates  [n_tokens][k] fp32 out.
 * Errors: EINVAL (null handle/pointer, n_tokens < 1 or > max_tokens), EHIP.
 * Asynchronous; may be called on its own (e.g. to prefetch for a later layer).
 */
int rvq_moe_route_topk(rvq_moe *h, const float *x, int32_t n_tokens, int32_t *ids, float *gates,
                       void *stream);

/*
 * rvq_moe_layer_forward -- y[t] = sum_j gates[t][j] * FFN_{ids[t][j]}(x_hat[t])
 * (+ x[t] when residual), FFN(v) = W_d (silu(W_g v) * (W_u v)).  Below the
 * chunk threshold it is evaluated from the codes by per-token tables of
 * partial dot products ([FR] "Quantification et exactitude"), fp32 throughout
 * (a batch is grouped by expert, so an expert's codes are read once per call).
 * At or above it (the chunk path, for prefill-sized calls) the tokens are
 * grouped by expert, the weights are rebuilt as bf16(c1 + c2 + c3) tile by
 * tile in registers, and x_hat and h are rounded to bf16 for bf16 x bf16 ->
 * fp32 matrix-core products: expect ~1e-3 relative error instead of ~1e-6.
 * With resident codes the chunk path runs the kernels of experts with more
 * than 32 tokens on a stream the handle owns, forked from `stream` after the
 * call's earlier work and joined back by events before anything enqueued on
 * `stream` later: the call is ordered as if all of it ran on `stream` (also
 * under stream capture).
 *   x      [n_tokens][d] fp32.   ids [n_tokens][k] int32.   gates [n_tokens][k] fp32.
 *   y      [n_tokens][d] fp32 out (must not alias x).
 * Ids outside [0, E) are detected on the device: the affected outputs are
 * unspecified and the error is returned by rvq_moe_sync / rvq_moe_close
 * (RVQ_MOE_EDEVICE).
 * Errors: EINVAL (null handle/pointer, n_tokens < 1 or > max_tokens, y == x), EHIP.
 */
int rvq_moe_layer_forward(rvq_moe *h, const float *x, int32_t n_tokens, const int32_t *ids,
                          const float *gates, float *y, void *stream);

/*
 * rvq_moe_layer_forward_noalloc -- rvq_moe_layer_forward's table path (per-token
 * tables of partial dot products, fp32) with no memory of the handle's
 * workspace and no allocation of any kind: for callers that cannot allocate
 * while they run (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The kernels' scratch -- gate/up partial
 * sums and inter-workgroup completion counters -- lives in one static device
 * array of 32 MiB per GPU (set up by the first rvq_moe_open on that GPU, held
 * until the process ends); its counters are cleared by a small kernel (no
 * memset) at the start of every call.  Every call on one GPU, from any
 * handle, shares that array: calls that overlap in time on one GPU race.
 * Same arguments, semantics and output as rvq_moe_layer_forward below its
 * chunk threshold (always the table path here, whatever n_tokens).
 *   Needs 2 * (n_tokens * top_k + 1) * 256 bytes of counters (rounded up to
 *   256) plus n_tokens * top_k * 2 * ceil(d / 256) * ceil(ffn / 32) * 128
 *   bytes of partial sums within the 32 MiB (d=7168, ffn=2048, top-16: up to
 *   4 tokens per call), and with `deterministic` also n_tokens * top_k *
 *   ceil(ffn / 256) * ceil(d / 32) * 128 bytes of output rows (up to 2 tokens
 *   per call at that shape).
 * Errors: EINVAL (as layer_forward; or a call that needs more scratch than the
 * array holds), ENOTSUP (streaming codes), EHIP.
 */
int rvq_moe_layer_forward_noalloc(rvq_moe *h, const float *x, int32_t n_tokens, const int32_t *ids,
                                  const float *gates, float *y, void *stream);

/*
 * rvq_moe_route_forward -- rvq_moe_route_topk and rvq_moe_layer_forward in one
 * launch: writes ids and gates (the same selection: top k of fp64 logits,
 * descending, ties to the lower id, softmax over the k) and y (the layer output
 * for them).  The logits' fp64 summation order differs from route_topk's, so
 * gates may differ from it in the last fp32 bit and near-ties (within ~1e-15
 * relative) may resolve differently.
 *   x [n_tokens][d] fp32; ids [n_tokens][k] int32 out; gates [n_tokens][k] fp32
 *   out; y [n_tokens][d] fp32 out (must not alias x).
 * Errors: EINVAL (null handle/pointer, n_tokens < 1 or > max_tokens,
 * n_tokens * top_k > 1024, y == x), ENOTSUP (streaming codes; or more than 4
 * experts per workgroup of the persistent grid, i.e. n_experts above 4 x the
 * device's resident workgroups -- 1024 on an MI355X), EHIP.
 */
int rvq_moe_route_forward(rvq_moe *h, const float *x, int32_t n_tokens, int32_t *ids, float *gates, float *y,
                          void *stream);

/*
 * rvq_moe_prefetch -- start making experts resident in the HBM slot cache of
 * a streaming handle (codes_location PINNED_HOST or PINNED_BANK) ahead of a later
 * layer_forward.  [FR] "Lecture anticipée et prédiction du routeur": the
 * router of the next layer, run on the current layer's hidden state, predicts
 * that layer's experts; the first 6 of its 16 are read early and consumed as
 * they land.  Typically `ids` come from rvq_moe_route_topk of THIS handle on
 * an earlier hidden state (any ids are accepted).
 *   ids        [n_tokens][k] int32, as route_topk writes them.
 *   per_token  how many leading ids of each token to prefetch, 1..k.
 * Synchronises `stream` once to read the ids on the host (as a streaming
 * layer_forward does), then enqueues the copies of the experts not resident
 * on the handle's copy stream, into least-recently-used slots (a slot still
 * read by an enqueued kernel is refilled only after that kernel); nothing
 * waits for them until a layer_forward uses their slots.  At most
 * cache_slots distinct experts are taken, in token-major order; ids outside
 * [0, E) are skipped.  Outputs of later calls do not depend on prefetching.
 * Errors: EINVAL (null handle/pointer, n_tokens < 1 or > max_tokens,
 * per_token outside 1..k), ENOTSUP (codes resident on the device), EHIP.
 */
int rvq_moe_prefetch(rvq_moe *h, const int32_t *ids, int32_t n_tokens, int32_t per_token, void *stream);

/*
 * rvq_moe_sync -- synchronise `stream`, then return any deferred device-side
 * error recorded by earlier calls: RVQ_MOE_ECORRUPT (a record check failed;
 * returned again by every later sync and by close) before RVQ_MOE_EDEVICE
 * (cleared once returned).
 */
int rvq_moe_sync(rvq_moe *h, void *stream);

/*
 * rvq_moe_close -- synchronise the device, free everything the handle owns,
 * and return any deferred device-side error.  NULL is accepted (returns OK).
 * [FR] "Objectif et forme d'implémentation de WASTE": the C API's exit call.
 */
int rvq_moe_close(rvq_moe *h);

/* Reason for the last failure on this thread (never NULL; "" if none). */
const char *rvq_moe_last_error(void);

/* Library ABI version (RVQ_MOE_ABI_VERSION of the built library). */
int rvq_moe_abi_version(void);

/* Per-handle counters, exact and host-side (no device readback). */
typedef struct rvq_moe_stats {
    uint64_t route_calls;
    uint64_t forward_calls;
    uint64_t tokens_routed;
    uint64_t tokens_forwarded;
    uint64_t expert_evals;          /* token x expert pairs evaluated */
    uint64_t code_bytes_resident;   /* bytes of the library's code copy (streaming: its HBM slots) */
    uint64_t record_bytes;          /* canonical bytes per expert record */
    uint64_t codebook_bytes;        /* bytes of one expert's codebooks */
    uint64_t h2d_bytes;             /* slot cache: bytes copied host -> HBM slots */
    uint64_t slot_hits;             /* slot cache: experts a call found resident */
    uint64_t slot_misses;           /* slot cache: experts copied in */
    uint64_t host_syncs;            /* slot cache: calls that read their ids back */
    uint64_t prefetch_fills;        /* slot cache: experts copied in by rvq_moe_prefetch */
    uint64_t prefetch_hits;         /* slot cache: of those, found resident by a later call */
    uint64_t records_checked;       /* slot cache: record copies followed by the trailer checks */
    uint64_t records_verified;      /* slot cache: of those, with the payload CRC-32 checked too */
} rvq_moe_stats;

int rvq_moe_get_stats(const rvq_moe *h, rvq_moe_stats *out);

/*
 * Kernel timing.  rvq_moe_set_profiling(h, every) makes every `every`-th
 * route_topk and every `every`-th layer_forward / route_forward call bracket its kernels with
 * HIP events on the caller's stream (0 disables).  rvq_moe_kernel_times
 * synchronises the device and returns, per kernel kind, the number of timed
 * launches and their summed duration in milliseconds, then clears the
 * samples; names[] receives static strings.  Returns the number of kinds
 * filled (>= 0) or a negative status.  Kinds:
 *   0 "route_topk"       the router and selection kernels of rvq_moe_route_topk,
 *   1 "layer_lut"        the persistent LUT kernel of rvq_moe_layer_forward,
 *   2 "route_layer_lut"  the persistent kernel of rvq_moe_route_forward.
 *   3 "chunk"            the chunk-path kernels of rvq_moe_layer_forward.
 */
#define RVQ_MOE_N_KERNEL_KINDS 4
int rvq_moe_set_profiling(rvq_moe *h, int every);
int rvq_moe_kernel_times(rvq_moe *h, const char **names, uint64_t *launches, double *total_ms,
                         int max_kinds);

#ifdef __cplusplus
}
#endif
#endif
