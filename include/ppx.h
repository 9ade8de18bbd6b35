/*
 * ppx.h -- C ABI of the MI355X (gfx950) pruned prompt-prefill engine.
 *
 * The engine runs the prompt-prefill forward pass of a Gemma-style decoder
 * whose layers from n_layer_kv_from_start on reuse, read-only, the KV cache
 * of an earlier layer.  Before the first such layer every token row except
 * the output row is pruned: an intermediate ubatch skips those layers and the
 * last ubatch carries one row through them ("llama.cpp Gemma 4 prefill KV
 * graph optimization", section 1).  A KV snapshot of the first N positions
 * can be saved and loaded so that a repeated prompt prefix resumes at N
 * ("PicoLM KV Cache persistence", sections on the cache flag, the file
 * contents and the load check).
 *
 * Conventions for every call:
 *  - Return value: PPX_OK (0) or a negative PPX_E_* status.  Nothing aborts
 *    and nothing prints unless the environment variable PPX_LOG is set.
 *  - Device pointers are HIP device memory of the current device; the caller
 *    owns them (KV buffer, workspace, logits) unless a call says otherwise.
 *  - hip_stream is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls are stream-ordered and asynchronous unless stated; argument
 *    checks happen synchronously, before any work is queued.
 *  - ppx_prefill runs one sequence (n_seq_max == 1), the case the pages
 *    prune; ppx_prefill_multi runs several, each in its own cache, with the
 *    prune generalised to one output row per sequence.
 *  - Host threads: a model keeps per-model state that its calls update (the
 *    recorded launch sequences, event pools, the tables' staging buffer), so
 *    calls on one model, or on caches of one model, come from one host
 *    thread at a time.  Different models are independent.
 */
#ifndef PPX_H
#define PPX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    PPX_OK = 0,
    PPX_E_INVAL = -1,       /* bad argument (NULL, size, alignment, params) */
    PPX_E_TOKEN = -2,       /* a token id outside [0, n_vocab)              */
    PPX_E_CTX = -3,         /* positions would exceed n_ctx                 */
    PPX_E_IO = -4,          /* file open/read/write failure                 */
    PPX_E_FORMAT = -5,      /* bad magic, version, truncated or bad sizes   */
    PPX_E_MISMATCH = -6,    /* snapshot layer count / kv dim != model       */
    PPX_E_UNSUPPORTED = -7, /* shape or option the engine does not support  */
    PPX_E_HIP = -8,         /* a HIP runtime call failed                    */
    PPX_E_NOMEM = -9,       /* buffer too small or device allocation failed */
    PPX_E_EMPTY = -10       /* n_tokens == 0: the last row must exist       */
};

typedef struct ppx_model ppx_model; /* library-owned: host state + device weights */
typedef struct ppx_kv ppx_kv;       /* handle over a caller-owned device KV buffer */

typedef struct {
    int n_layer;               /* L                                           */
    int n_layer_kv_from_start; /* Ls: layers [0, Ls) own KV, [Ls, L) share    */
    int d_model, n_head, n_kv_head, head_dim, n_ff, n_vocab;
    int ple_dim;               /* per-layer embedding width E (0 = none)      */
    int kv_dim;                /* n_kv_head * head_dim                        */
    int act;                   /* 0 GeGLU, 1 SwiGLU                           */
    int has_nextn;             /* 1: the container holds a next-n head        */
} ppx_model_info;

enum { PPX_PRUNE_AUTO = -1, PPX_PRUNE_OFF = 0, PPX_PRUNE_ON = 1 };

/* Per-phase kernel timing of one prefill call (see ppx_prefill_params). */
enum { PPX_PHASE_GEMM = 0,    /* Q4_0 MFMA GEMMs of the row-batched layers      */
       PPX_PHASE_ATTN = 1,    /* causal prefill attention                        */
       PPX_PHASE_ROW = 2,     /* single-row path: GEMVs, 1-row attention, norms  */
       PPX_PHASE_OTHER = 3,   /* embedding gather, row norms, copies             */
       PPX_N_PHASES = 4 };
typedef struct {
    double ms[PPX_N_PHASES];   /* summed event time around each phase's launches */
    int launches[PPX_N_PHASES];
    double gemm_flop;          /* algorithmic 2*M*N*K over the GEMM launches      */
    double attn_flop;          /* 4*n_head*head_dim*(visible keys) over queries   */
    double row_bytes;          /* Q4_0 weight bytes + KV bytes the row path reads */
    double glu_ms;             /* the gate|up GEMM launches alone (also in GEMM)  */
    int glu_launches;
    double glu_flop;           /* their algorithmic 2*M*N*K                       */
} ppx_timing;

typedef struct {
    int n_ubatch;   /* rows per ubatch, 1..PPX_MAX_UBATCH; must not exceed the
                       n_ubatch given to ppx_workspace_bytes                    */
    int prune;      /* PPX_PRUNE_AUTO: the predicate decides; OFF: every row
                       through every layer; ON: PPX_E_UNSUPPORTED if the
                       predicate is false                                       */
    int embeddings; /* 1: write every row's output-normed final hidden state to
                       embd_out (the predicate then forbids pruning)            */
    int n_seq_max;  /* ppx_prefill: must be 1; ppx_prefill_multi: >= n_seq    */
    float *debug_hidden; /* NULL, or device fp32 [n_layer][d_model]: receives
                            the last row's hidden state after each layer       */
    ppx_timing *timing;  /* NULL, or host struct filled with per-phase kernel
                            times; HIP events are then recorded around every
                            launch and the call synchronises the stream        */
    float *debug_rows;   /* NULL, or device fp32 [n_layer][n_tokens][d_model]:
                            receives the hidden state entering each layer for
                            every row that layer processes (pruned layers: the
                            last row only; other entries are left untouched)    */
    const uint8_t *embeddings_layer_inp; /* NULL (none), or host flags
                            [n_layer + 1]: flag il requests every row's hidden
                            state entering layer il (il = n_layer: the final
                            hidden state before the output norm); the
                            predicate forbids pruning when a flag at
                            il >= n_layer_kv_from_start is set              */
    float *layer_inp_out; /* device fp32 [n_flagged][n_tokens][d_model]: the
                            flagged layers' inputs in increasing layer order;
                            required when any flag is set                    */
    float *embd_out;     /* device fp32 [n_tokens][d_model]: required when
                            embeddings != 0                                  */
    int precision;       /* PPX_PRECISION_FAST (0, the default) or
                            PPX_PRECISION_EXACT; see below                   */
    float *nextn_logits; /* NULL, or device fp32 [n_vocab]: the next-n head's
                            logits (see below); requesting them makes the
                            predicate's crop_before_nextn false            */
} ppx_prefill_params;

/* Arithmetic of the row-batched layers (the single-row path and the head
 * are fp32-class in both):
 *  - FAST: fp16 MFMA operands with fp32 accumulation -- activations, the
 *    attention query, probabilities and output rounded to fp16, weights
 *    entering the products as fp16(d * (code - 8)); the K|V projection
 *    alone uses exact weights and split activations.
 *  - EXACT: every product at ~fp32 accuracy -- each fp32 operand split into
 *    fp16 high and low parts against exact (code - 8) weights, each 32-wide
 *    block's partial scaled by its fp32 block scale; attention of every row
 *    in fp32 (online softmax over 32-key chunks, both products split the same
 *    way).  Several times slower; for models whose activations amplify fp16
 *    rounding beyond the tolerance a comparison needs. */
enum { PPX_PRECISION_FAST = 0, PPX_PRECISION_EXACT = 1 };

/* Next-n head.  The llama.cpp Gemma 4 prefill page (section 1) lets the prune
 * apply only when the output rows can be cropped before a next-n head, i.e.
 * no such head reads another row.  A container may hold one (F32 tensor
 * "nextn_norm" [1][d_model]); it is a depth-1 multi-token predictor that
 * shares the output matrix:
 *     z      = x_{n-2} + embd_scale * deq(tok_embd[id_{n-1}])
 *     logits = W_out rms(z, nextn_norm)
 * where x_{n-2} is the final hidden state (before the output norm) of the
 * call's second-to-last row and id_{n-1} the last token.  It needs a row the
 * prune drops, so a call that requests it runs every row through every
 * layer (prune AUTO turns it off; ON gives PPX_E_UNSUPPORTED).  Requires
 * n_tokens >= 2 (PPX_E_INVAL) and a model with the head (PPX_E_UNSUPPORTED);
 * ppx_prefill_multi does not serve it (PPX_E_UNSUPPORTED). */

#define PPX_MAX_UBATCH 4096
#define PPX_MAX_SEQ 64

/* ---------------------------------------------------------------- model */

/* Load a "PPXM" v1 container (Q4_0 weights, fp32 norm gains; layout in the
 * synthetic-input module's docstring) from host memory.  The bytes are read
 * during the call only.  Weights are repacked for the kernels and uploaded
 * into device memory the library allocates (freed by ppx_model_free).
 * Errors: PPX_E_FORMAT (bad container), PPX_E_UNSUPPORTED (a dimension the
 * kernels cannot tile: d_model, q_dim, n_ff, ple_dim not multiples of 256,
 * head_dim not 64/128/256, n_head not a multiple of n_kv_head), PPX_E_HIP. */
int ppx_model_load(const void *container, size_t bytes, void *hip_stream, ppx_model **out);
/* Same, reading the container from a file (PPX_E_IO if it cannot be read). */
int ppx_model_load_file(const char *path, void *hip_stream, ppx_model **out);
/* Device bytes the repacked weights of a container need (host only: the
 * container is parsed and laid out, nothing touches the GPU); 0 if the
 * container is invalid or unsupported. */
size_t ppx_model_weight_bytes(const void *container, size_t bytes);
/* As ppx_model_load, with the repacked weights placed in caller-owned device
 * memory (a torch tensor, say): weights_dev 256-byte aligned, weights_bytes
 * >= ppx_model_weight_bytes.  The buffer must outlive the model and is not
 * freed by ppx_model_free; the library still allocates the small RoPE table
 * of each context length it meets.  Errors: those of ppx_model_load, and
 * PPX_E_INVAL (NULL or misaligned weights_dev), PPX_E_NOMEM (too small). */
int ppx_model_load_into(const void *container, size_t bytes, void *weights_dev, size_t weights_bytes,
                        void *hip_stream, ppx_model **out);
void ppx_model_free(ppx_model *m);
int ppx_model_get_info(const ppx_model *m, ppx_model_info *out);
/* Device bytes of the model's repacked weights (the library's allocation, or
 * the part of the caller's buffer in use after ppx_model_load_into). */
size_t ppx_model_device_bytes(const ppx_model *m);

/* ---------------------------------------------------------------- KV cache */

/* fp16 K and V of the Ls owning layers: K as [Ls][n_ctx][kv_dim] first (its
 * size rounded up to 256 bytes), then V transposed, [Ls][kv_dim][vld] with
 * vld = n_ctx rounded up to a multiple of 64 (values of consecutive positions
 * contiguous, as the attention kernels read them). */
size_t ppx_kv_bytes(const ppx_model *m, int n_ctx);
/* Wrap a caller-owned device buffer of >= ppx_kv_bytes bytes (256-byte
 * aligned) as an empty cache (n_pos = 0).  The buffer must outlive the
 * handle; ppx_kv_free releases the handle only.  Zeroes the buffer and
 * builds the model's RoPE tables up to n_ctx if they are shorter (blocking). */
int ppx_kv_init(ppx_model *m, void *kv_dev, size_t bytes, int n_ctx, ppx_kv **out);
void ppx_kv_free(ppx_kv *kv);
int ppx_kv_n_pos(const ppx_kv *kv);
int ppx_kv_n_ctx(const ppx_kv *kv);
/* Forget all positions (n_pos = 0); the buffer contents are left as is. */
int ppx_kv_clear(ppx_kv *kv);

/* KVCP snapshot ("PicoLM KV Cache persistence", file-content section):
 * "KVCP", int32 n_pos, int32 n_layers (= Ls), int32 kv_dim, then K as
 * [n_layers][n_pos][kv_dim] fp16, then V likewise; little-endian.
 * kv_save writes the first n_pos (<= ppx_kv_n_pos) positions and
 * synchronises hip_stream.  kv_load checks the file before touching the
 * cache (magic, layer count, kv dim, exact size -- the KVCP body, or the body
 * and a token section as written by ppx_kv_save_tokens --, n_pos <= file positions,
 * n_pos <= n_ctx); on any failure it returns PPX_E_FORMAT / PPX_E_MISMATCH /
 * PPX_E_CTX / PPX_E_IO and leaves the cache empty (n_pos = 0), so the caller
 * falls back to a full prefill.  On success n_pos = the loaded count; it
 * synchronises hip_stream.  The file stores no token ids: that the new
 * prompt starts with the cached prefix is the caller's duty (see
 * ppx_kv_save_tokens / ppx_kv_load_prefix for a checked variant). */
int ppx_kv_save(const ppx_kv *kv, const char *path, int n_pos, void *hip_stream);
int ppx_kv_load(ppx_kv *kv, const char *path, int n_pos, void *hip_stream);

/* Token-verified prefix reuse (an extension outside the KVCP layout of the
 * PicoLM page, whose invalidation rules leave prefix checking to the
 * caller).  ppx_kv_save_tokens writes the same KVCP body as ppx_kv_save and
 * then a token section: "KVTK", int32 count (= n_pos), and the n_pos int32
 * token ids (host array) of the cached positions.  ppx_kv_load and
 * ppx_kvfile_validate accept such a file (the body is unchanged).
 * ppx_kv_load_prefix reads a file with a token section, takes the longest
 * common prefix L of its ids and tokens_host[0..n_tokens), capped at
 * n_tokens - 1 (so at least one token is left to prefill, which yields the
 * logits) and at n_ctx, loads the first L positions as ppx_kv_load(kv, path,
 * L) does, and stores L in *n_reused; the caller then prefills
 * tokens_host[L..n_tokens).  L = 0 loads nothing and returns PPX_OK.  Errors
 * leave the cache empty (n_pos = 0) and *n_reused = 0: PPX_E_FORMAT (no
 * token section, or the checks of ppx_kv_load), PPX_E_MISMATCH, PPX_E_IO,
 * PPX_E_INVAL (null arguments). */
int ppx_kv_save_tokens(const ppx_kv *kv, const char *path, int n_pos, const int32_t *tokens_host, void *hip_stream);
int ppx_kv_load_prefix(ppx_kv *kv, const char *path, const int32_t *tokens_host, int n_tokens, int *n_reused,
                       void *hip_stream);
/* Host-only check of a KVCP file against a model shape, the same check
 * ppx_kv_load makes before touching the cache: PPX_OK if the file is a
 * whole snapshot with n_layers layers of width kv_dim holding at least n_pos
 * positions and n_pos <= n_ctx; *file_n_pos (if not NULL) receives the
 * file's position count whenever the header could be read. */
int ppx_kvfile_validate(const char *path, int n_layers, int kv_dim, int n_pos, int n_ctx, int *file_n_pos);

/* ---------------------------------------------------------------- prefill */

/* Device workspace bytes one prefill needs for ubatches of up to n_ubatch
 * rows and prompts of up to n_ctx tokens. */
size_t ppx_workspace_bytes(const ppx_model *m, int n_ubatch, int n_ctx);

/* Run tokens_host[0..n_tokens) at positions n_pos .. n_pos+n_tokens-1 of kv
 * and write the logits of the last token, fp32 [n_vocab], to logits_dev.
 * KV-owning layers write their fp16 K/V at those positions; KV-shared layers
 * read their source layer's cache and write nothing.  ws_dev (>=
 * ppx_workspace_bytes, 256-byte aligned) is scratch for the call.  On
 * success kv's n_pos advances by n_tokens.  Errors are reported before any
 * work is queued and leave n_pos unchanged: PPX_E_EMPTY, PPX_E_TOKEN,
 * PPX_E_CTX, PPX_E_INVAL (also: an extraction without its output buffer),
 * PPX_E_UNSUPPORTED (prune ON while the predicate is false, n_seq_max !=
 * 1), PPX_E_NOMEM (ws too small); PPX_E_HIP if a launch fails.
 * Extraction (embeddings, embeddings_layer_inp): the prune predicate of the
 * llama.cpp Gemma 4 prefill page, section 1, is evaluated with the call's
 * flags, so extracting the embeddings or a layer from the first KV-shared
 * one on runs every row through every layer, while extracting only earlier
 * layers keeps the prune.  The host token array is copied during the call.
 * One call in flight per kv. */
int ppx_prefill(ppx_model *m, ppx_kv *kv, const int32_t *tokens_host, int n_tokens,
                const ppx_prefill_params *p, void *ws_dev, size_t ws_bytes, float *logits_dev,
                void *hip_stream);

/* One prompt of a multi-sequence prefill: tokens_host[0..n_tokens) run at
 * positions kv->n_pos .. in kv, a cache no other sequence of the call uses. */
typedef struct {
    ppx_kv *kv;
    const int32_t *tokens_host;
    int n_tokens;
} ppx_seq;

/* Device workspace bytes of a ppx_prefill_multi call over n_seq prompts of
 * n_tokens_total tokens together, in caches of up to n_ctx_max positions;
 * 0 for arguments out of range. */
size_t ppx_workspace_bytes_multi(const ppx_model *m, int n_ubatch, int n_seq, long n_tokens_total, int n_ctx_max);

/* Several independent prompts in one pass (1 <= n_seq <= PPX_MAX_SEQ,
 * n_seq <= p->n_seq_max); row s of logits_dev (fp32 [n_seq][n_vocab])
 * receives the logits of prompt s's last token, and each sequence's result
 * is that of ppx_prefill of its prompt alone.  The rows of all prompts are
 * laid end to end and cut into ubatches of p->n_ubatch rows, so short
 * prompts share the row-batched GEMMs; each row writes K/V into, and attends
 * over, its own sequence's cache.  Pruning (the llama.cpp Gemma 4 prefill
 * page, section 1, excludes several sequences at merge time; this is the
 * generalisation to one output row per sequence): before the first KV-shared
 * layer the last row of every prompt is gathered, and those n_seq rows alone
 * run the KV-shared layers, each reading its own sequence's source-layer
 * cache, and the head.  p->prune AUTO / ON apply the predicate with the
 * sequence-count clause taken per sequence.  n_seq == 1 is ppx_prefill.
 * ws_dev: >= ppx_workspace_bytes_multi bytes, 256-byte aligned.  On success
 * every kv's n_pos advances by its n_tokens.  Errors are reported before any
 * work is queued and leave every n_pos unchanged: PPX_E_EMPTY (a prompt of
 * no tokens), PPX_E_TOKEN, PPX_E_CTX, PPX_E_INVAL (NULL arguments, a cache
 * used twice or built for another model, n_seq out of range), PPX_E_UNSUPPORTED
 * (extraction, debug outputs, prune ON while the predicate is false),
 * PPX_E_NOMEM; PPX_E_HIP if a launch fails.  The host token arrays are read
 * during the call; the call may wait for the previous multi-sequence call of
 * the same model to have copied its tables.  One call in flight per kv. */
int ppx_prefill_multi(ppx_model *m, const ppx_seq *seqs, int n_seq, const ppx_prefill_params *p, void *ws_dev,
                      size_t ws_bytes, float *logits_dev, void *hip_stream);

/* ---------------------------------------------------------------- unified cache
 *
 * One KV buffer shared by several sequences (the llama.cpp Gemma 4 prefill
 * page, section 5, measures such a unified cache against one cache per
 * sequence).  Every cell holds one position of one sequence; cells are handed
 * out in pages of 64 consecutive positions of one sequence, the lowest free
 * page first, so a sequence that grows over several calls holds pages
 * scattered through the buffer, and a row attends only to the cells of its
 * own sequence up to its position.  The layout per KV-owning layer is that of
 * ppx_kv with n_cells in place of n_ctx (K [n_cells][kv_dim], V transposed
 * [kv_dim][n_cells]). */
typedef struct ppx_kvu ppx_kvu;

/* Device bytes of a unified cache of n_cells cells (a positive multiple of
 * 64); 0 otherwise. */
size_t ppx_kvu_bytes(const ppx_model *m, int n_cells);
/* Wrap caller-owned device memory (>= ppx_kvu_bytes, 256-byte aligned; the
 * caller frees it after ppx_kvu_free) as a unified cache for sequence ids
 * 0 .. n_seq_max - 1 (1 <= n_seq_max <= 65536), all empty.  PPX_E_INVAL,
 * PPX_E_NOMEM (bytes too small), PPX_E_HIP. */
int ppx_kvu_init(ppx_model *m, void *kv_dev, size_t bytes, int n_cells, int n_seq_max, ppx_kvu **out);
void ppx_kvu_free(ppx_kvu *u);
/* Positions held by sequence seq_id (PPX_E_INVAL for a bad id or handle). */
int ppx_kvu_n_pos(const ppx_kvu *u, int seq_id);
/* Cells in pages that no sequence holds. */
int ppx_kvu_free_cells(const ppx_kvu *u);
/* Release every cell of sequence seq_id (its n_pos becomes 0).  The cells'
 * contents stay until a later call overwrites them; no kernel reads them.
 * Host-only: the caller orders it after any queued call that uses them. */
int ppx_kvu_seq_rm(ppx_kvu *u, int seq_id);
/* The cell of each of positions 0 .. n-1 of sequence seq_id, into
 * cells_host[0..n) (host int32); n <= ppx_kvu_n_pos.  PPX_E_INVAL. */
int ppx_kvu_cells(const ppx_kvu *u, int seq_id, int32_t *cells_host, int n);

/* One prompt of a unified-cache prefill: tokens_host[0..n_tokens) of
 * sequence seq_id, continuing at that sequence's position count. */
typedef struct {
    int seq_id;
    const int32_t *tokens_host;
    int n_tokens;
} ppx_useq;

/* Device workspace bytes of a ppx_prefill_unified call over n_seq prompts of
 * n_tokens_total tokens together in a cache of n_cells cells; 0 for
 * arguments out of range. */
size_t ppx_workspace_bytes_unified(const ppx_model *m, int n_ubatch, int n_seq, long n_tokens_total, int n_cells);

/* ppx_prefill_multi over one unified cache: prompt s (distinct seq_ids)
 * takes the free pages its new positions need, then the pass is that of
 * ppx_prefill_multi (rows end to end in ubatches, the same generalised prune,
 * one logits row per prompt) with every K/V write and read going to the
 * sequence's cells.  Each sequence's result equals ppx_prefill of its prompt
 * alone in a cache of its own; n_seq == 1 runs the same pass.  A generation
 * step is a call with one token.  Errors are reported before any work is
 * queued and leave every sequence and page unchanged: PPX_E_EMPTY,
 * PPX_E_TOKEN, PPX_E_CTX (a sequence past n_cells positions, or too few free
 * pages), PPX_E_INVAL (NULL arguments, a seq_id out of range or repeated, a
 * cache of another model), PPX_E_UNSUPPORTED (extraction, debug outputs, the
 * next-n head, prune ON while the predicate is false), PPX_E_NOMEM; PPX_E_HIP
 * if a launch fails.  Asynchronous on the stream; one call in flight per
 * cache. */
int ppx_prefill_unified(ppx_model *m, ppx_kvu *u, const ppx_useq *seqs, int n_seq, const ppx_prefill_params *p,
                        void *ws_dev, size_t ws_bytes, float *logits_dev, void *hip_stream);

/* One generation step after a prefill: the row of `token` at position n_pos
 * runs through every layer on the single-row (GEMV) path -- KV-owning layers
 * append its fp16 K and V at n_pos, KV-shared layers read their source
 * layer's cache -- and the logits of that row, fp32 [n_vocab], go to
 * logits_dev.  The result is that of ppx_prefill of the one token (the
 * pages' text-generation runs, "tg128", reuse the same cache after a
 * prefill).  ws_dev: >= ppx_workspace_bytes(m, 1, n_ctx) bytes (a prefill's
 * workspace for the same n_ctx is large enough), 256-byte aligned.  On
 * success n_pos advances by one.  Errors are reported before any work is
 * queued and leave n_pos unchanged: PPX_E_TOKEN, PPX_E_CTX (cache full),
 * PPX_E_INVAL, PPX_E_NOMEM; PPX_E_HIP if a launch fails.  Asynchronous on
 * the stream; one call in flight per kv. */
int ppx_decode(ppx_model *m, ppx_kv *kv, int32_t token, void *ws_dev, size_t ws_bytes, float *logits_dev,
               void *hip_stream);

/* ppx_decode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc): the same kernels run in a scratch array of
 * ppx_decode_static_limit() bytes (32 MiB) that the library holds on every
 * GPU it runs on until the process ends.  The call allocates nothing.  It
 * returns PPX_E_NOMEM when the cache's context needs more scratch than that
 * (ppx_workspace_bytes(m, 1, n_ctx) > the limit), PPX_E_HIP if the array's
 * address cannot be looked up, and otherwise behaves as ppx_decode.  Every
 * call on one GPU shares that GPU's array and leaves its contents behind:
 * calls that overlap on one GPU (other host threads, other streams) race
 * and must be serialised by the caller. */
int ppx_decode_static(ppx_model *m, ppx_kv *kv, int32_t token, float *logits_dev, void *hip_stream);
size_t ppx_decode_static_limit(void);

/* The prune predicate printed on the llama.cpp Gemma 4 prefill page
 * (section 1): 1 iff crop_before_nextn, 0 < n_layer_kv_from_start < n_layer,
 * !embeddings, n_seq_max == 1 and no embeddings_layer_inp[il] is set for il
 * in [n_layer_kv_from_start, n_layer] (n_layer + 1 flags; NULL = none). */
int ppx_prune_predicate(int n_layer, int n_layer_kv_from_start, int embeddings, int n_seq_max,
                        const uint8_t *embeddings_layer_inp, int crop_before_nextn);

/* ---------------------------------------------------------------- kernel-level entry points
 * These expose single kernels of the prefill path so that each can be
 * checked against the oracle at full model shapes.  Tensors are named as in
 * the container ("blk.3.ffn_down", "tok_embd", ...); fused tensors are
 * addressed by their first member: "blk.3.wq" = Q rows in RoPE-pair order
 * (16-row blocks alternate the two halves of each head), "blk.3.wk" = K
 * rows in that order followed by V rows (owning layers), "blk.3.ffn_gate" =
 * gate|up with 8-row blocks alternating gate and up.
 *
 * fp16 activations that feed a GEMM (and the prefill attention's output)
 * use the engine's fragment-tiled layout: A[M][K] is cut into 16-row x
 * 32-column tiles of 1 KB stored tile-row-major, and inside a tile element
 * (r, k) sits at lane * 8 + k % 8 with lane = r % 16 + 16 * ((k % 32) / 8).
 * A tiled [M][K] buffer holds ceil(M/16)*16 rows; ppx_op_tile_f16 converts
 * from row-major. */

/* Row-major fp16 [M][K] -> fragment-tiled (K % 32 == 0); dst holds
 * ceil(M/16)*16 rows, of which the padding rows are left untouched. */
int ppx_op_tile_f16(const void *src_dev, int M, int K, void *dst_dev, void *hip_stream);

/* Read bytes (a positive multiple of 1024) of device memory at src_dev
 * (16-byte aligned) through LDS DMA -- the load instruction and the 1 KB
 * per-wave pattern with which the GEMM's producer waves fetch their operands
 * -- over n_workgroups workgroups (1..65536) of four waves; workgroup w
 * writes the XOR of the 32-bit words it read to xor_dev[w] (device uint32
 * [n_workgroups]), so the XOR over all of them is that of the buffer.  For
 * calibrating hardware byte counters against a known byte count.
 * PPX_E_INVAL for bad arguments. */
int ppx_op_stream_read(const void *src_dev, size_t bytes, uint32_t *xor_dev, int n_workgroups, void *hip_stream);

/* Dequantise a whole Q4_0 tensor from the engine's repacked device layout
 * into fp32 [rows][cols] row-major (exact). */
int ppx_op_dequant(const ppx_model *m, const char *tensor, float *out_dev, void *hip_stream);
/* Bytes of scratch ppx_op_gemm / ppx_op_gemm_glu use for an M-row product
 * with the named tensor when K is split over workgroups (fp32 partial tiles,
 * summed in split order by a second kernel); 0 when that shape is not split. */
size_t ppx_op_gemm_workspace_bytes(const ppx_model *m, const char *tensor, int M);
/* C[M][N] (fp32, ldc = N) = A[M][K] (fp16, fragment-tiled) x W^T on the
 * MFMA GEMM path, W = the named container tensor [N][K].  ws_dev: scratch of
 * ppx_op_gemm_workspace_bytes bytes, or NULL (the product then runs without
 * the split; results are equal up to the order of the fp32 sums). */
int ppx_op_gemm(const ppx_model *m, const char *tensor, const void *a_dev_f16, int M, float *c_dev,
                void *ws_dev, size_t ws_bytes, void *hip_stream);
/* The gate|up GEMM of a layer with its fused activation epilogue, exactly
 * as the prefill runs it for the row-batched layers (the GeGLU feed-forward
 * of the Gemma-style decoder of "llama.cpp Gemma 4 prefill KV graph
 * optimization"; SwiGLU for a model whose activation is SwiGLU):
 * h[M][F] (fp16, fragment-tiled) = act(A Wg^T) * (A Wu^T), A fp16 [M][K]
 * fragment-tiled.  `tensor` must be a fused gate|up name ("blk.i.ffn_gate");
 * PPX_E_INVAL otherwise.  ws_dev as for ppx_op_gemm.  Asynchronous on the
 * stream. */
int ppx_op_gemm_glu(const ppx_model *m, const char *tensor, const void *a_dev_f16, int M, void *h_dev_f16,
                    void *ws_dev, size_t ws_bytes, void *hip_stream);
/* The same on the exact-weight path used for the fused K|V weight
 * ("blk.i.wk", owning layers): A = a_hi + a_lo (two fp16 [M][K] arrays,
 * fragment-tiled),
 * weights (code - 8) exactly with the fp32 block scale applied per 32-block. */
int ppx_op_gemm_exact(const ppx_model *m, const char *tensor, const void *a_hi, const void *a_lo, int M,
                      float *c_dev, void *hip_stream);
/* y[N] (fp32) = W x on the single-row (GEMV) path; x fp32 [K]. */
int ppx_op_gemv(const ppx_model *m, const char *tensor, const float *x_dev, float *y_dev,
                void *hip_stream);
/* Causal prefill attention: q fp16 [M][n_head][head_dim] at positions
 * pos0..pos0+M-1 over k fp16 [>= pos0+M][n_kv_head][head_dim] and the values
 * in the cache's transposed layout, vt fp16 [n_kv_head][head_dim][vld]
 * (vld a multiple of 64, >= pos0+M); o fp16 [M][n_head*head_dim]
 * fragment-tiled (the O projection's operand).  ws_dev is
 * scratch of ppx_workspace_bytes(m, M, pos0+M) bytes (1 <= M <= PPX_MAX_UBATCH). */
int ppx_op_attention(const ppx_model *m, const void *q_dev, const void *k_dev, const void *vt_dev,
                     int vld, int M, int pos0, void *o_dev, void *ws_dev, size_t ws_bytes, void *hip_stream);
/* Single-query attention: q fp32 [n_head][head_dim] at position pos over the
 * first pos+1 cache positions (k as above, vt transposed with vld > pos, a
 * multiple of 64); o fp32 [n_head*head_dim].  ws_dev is scratch of
 * ppx_workspace_bytes(m, 1, pos+1) bytes. */
int ppx_op_attention_1row(const ppx_model *m, const float *q_dev, const void *k_dev,
                          const void *vt_dev, int vld, int pos, float *o_dev, void *ws_dev, size_t ws_bytes,
                          void *hip_stream);

const char *ppx_status_str(int status);

#ifdef __cplusplus
}
#endif
#endif /* PPX_H */
