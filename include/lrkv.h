/*
 * lrkv.h - C ABI of the LRKV library: Low-Rank Key Value attention decode read straight
 * from a factored paged KV cache, on AMD Instinct MI355X (gfx950, CDNA4).
 *
 * Source of the method: the web page "Low-Rank Key Value Attention｜共享缓存与逐头残差"
 * (Zhongzhu Zhou's reading notes on arXiv 2601.11471), called "LRKV notes" below.
 *
 * Each layer has one shared key projection and one shared value projection, and every head
 * h adds a rank-r residual to each:  W_h = W_S + U_h B_h^T  (LRKV notes §3, eq 2-5).  For a
 * token x the cache keeps the shared rows S_K = x W_S_K, S_V = x W_S_V (width d_h) once, and
 * per head the private rows R_K[h] = x U_K[h], R_V[h] = x U_V[h] (width r).  The per-head
 * bases B_K[h], B_V[h] stay weights.  Full per-head keys and values are never formed.
 *
 * ---------------------------------------------------------------------------------------
 * Factored page layout (one page table for shared and private rows: LRKV notes §3, the
 * paragraph after Algorithm 1 asking that both kinds of page share token numbering and
 * lifetime).
 *
 *   P   = page_size tokens per page (16 for every compiled variant)
 *   b   = element bytes (4 for LRKV_F32, 2 for LRKV_BF16)
 *   C   = 16 / b elements per 16-byte chunk; d_h and r must be multiples of C
 *   page_bytes = P * 2 * (d_h + H*r) * b     (eq 9 of LRKV notes §4, per page)
 *
 * A page is four sections, in this order (element offsets from the page start):
 *   S_K          at 0                         P x d_h elements
 *   S_V          at P*d_h                     P x d_h
 *   R_K[h]       at 2*P*d_h + h*P*r           P x r, for h = 0..H-1
 *   R_V[h]       at 2*P*d_h + H*P*r + h*P*r   P x r, for h = 0..H-1
 * Inside each section (width w = d_h or r) feature k of token slot t sits at element
 *   ((k / C) * P + t) * C + (k % C)
 * i.e. chunk-major: the 16-byte chunk column c holds the P tokens' features [cC, cC+C)
 * back to back.  One 1 KiB load of a wavefront then hands lane (c, t) one token's chunk.
 *
 * With key_norm = 1 a fifth section follows R_V (LRKV notes §8, RMSNorm paragraph):
 *   N[h]         at 2*P*d_h + 2*H*P*r + h*P   P elements: 1/n of head h for slots 0..P-1
 * and the page is padded to a multiple of 1024 bytes (page_bytes = the sections' bytes
 * rounded up; the padding is never read or written): a page starting off a 1 KiB boundary
 * reads markedly slower.  Pages of the other layouts are whole KiB already (P = 16).
 *
 * Grouped pages (LRKV notes §3, after the gradient formulas: one shared block per group of
 * heads, groups = G > 1, H a multiple of G): head h belongs to group g = h / (H/G) and uses
 * that group's shared rows S_K[g], S_V[g].  A page is G blocks in group order, block g laid
 * out exactly like a one-group page of the group's H/G heads (S_K[g], S_V[g], then R_K and
 * R_V of heads g*H/G .. (g+1)*H/G - 1); page_bytes = P * 2 * (G*d_h + H*r) * b.
 *
 * Token position j of request b lives in page page_table[b * max_pages_per_req + j / P],
 * slot j % P, in all sections.  Page ids index a pool of num_pages * page_bytes bytes.
 *
 * ---------------------------------------------------------------------------------------
 * Conventions for every entry point:
 *  - Pointers marked "device" are HIP device pointers (hipMalloc / torch CUDA tensors);
 *    all must be 16-byte aligned.  Pointers to lrkv_layout are host pointers.
 *  - The caller owns every buffer (pool, page table, lengths, workspace, output).  The
 *    library never allocates or frees memory and keeps no state between calls; calls are
 *    re-entrant and thread-safe.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and is
 *    asynchronous; the library never synchronizes.  Calls that share a workspace or write
 *    the same pool rows must be ordered by the caller (one stream does that).
 *  - Every argument check runs on the host before any launch.  Values that live in device
 *    memory (page ids, lengths, row positions) are not checked by lrkv_append and
 *    lrkv_decode: out-of-range values are undefined behaviour.  lrkv_check_indices counts
 *    them on the device for a caller who wants to validate first.
 *  - Return value: LRKV_OK, or a negative status (lrkv_status_string gives its text).
 *
 * Shapes with a compiled kernel variant, (H, d_h, r, dtype):
 *   (4, 16, 4, LRKV_F32), (16, 128, 56, LRKV_BF16), (32, 128, 32, LRKV_BF16); P = 16;
 *   the two bf16 shapes also with key_norm = 1 (their multi-query calls then run through
 *   the split decode kernels rather than the prefill kernel); (32, 128, 32, LRKV_BF16)
 *   also with groups = 2 (lrkv_append and lrkv_decode; multi-query calls through the split
 *   kernels).
 * Any other shape returns LRKV_ERR_UNSUPPORTED.
 */
#ifndef LRKV_H
#define LRKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { LRKV_F32 = 0, LRKV_BF16 = 1 };

enum {
  LRKV_OK = 0,
  LRKV_ERR_INVALID_ARG = -1, /* null / misaligned pointer, bad size, workspace too small */
  LRKV_ERR_UNSUPPORTED = -2, /* (H, d_h, r, dtype, P) without a kernel variant          */
  LRKV_ERR_HIP = -3,         /* the HIP runtime reported an error at launch            */
  LRKV_ERR_SCRATCH = -4,     /* lrkv_decode_noalloc: the call needs more than its fixed */
                             /* scratch holds                                           */
  LRKV_ERR_NO_PAGES = -5     /* the page pool has fewer free pages than asked for       */
};

/* Description of the cache.  Physical rank = logical rank: no padding of r (LRKV notes §4
 * asks that a padded physical width be recorded apart from the logical rank; this layout
 * has none). */
typedef struct lrkv_layout {
  int32_t num_heads; /* H   */
  int32_t head_dim;  /* d_h */
  int32_t rank;      /* r   */
  int32_t page_size; /* P   */
  int32_t dtype;     /* LRKV_F32 or LRKV_BF16 */
  int32_t key_norm;  /* 0, or 1: pages keep the key-norm section N (see lrkv_key_norms) */
  int32_t groups;    /* shared blocks G (0 or 1: one for all heads); see "Grouped pages" */
} lrkv_layout;

/* Bytes of one page: P * 2 * (d_h + H*r) * b, plus P * H * b with key_norm.  With P tokens
 * the dense multi-head cache would take P * 2 * H * d_h * b, so page_bytes over that is
 * exactly 1/H + r/d_h (LRKV notes §4, eq 9), plus 1/(2 d_h) with key_norm (§8).  Returns 0
 * if L is NULL or describes no valid layout. */
size_t lrkv_page_bytes(const lrkv_layout* L);

/* Algorithm 1 of LRKV notes §3: build or append the factored cache.
 *
 * For each new row n (0 <= n < n_rows) computes, with float32 accumulation,
 *   S_K = X[n] W_SK,  S_V = X[n] W_SV,  R_K[h] = X[n] U_K[:, h, :],  R_V[h] = X[n] U_V[:, h, :]
 * rounds each value to nearest even in L->dtype and writes it at position row_pos[n] of
 * request row_req[n], i.e. page page_table[row_req[n] * max_pages_per_req + row_pos[n]/P],
 * slot row_pos[n] % P, in the four sections.  No other byte of the pool changes.  Prefill
 * (all rows of a prompt) and single-token append are the same call.
 *
 * WEIGHT ORIENTATION - read this before passing weights.  The page writes the products as
 * X W_S with W_S of shape [d][d_h] and X U_h with U_h of shape [d][r].  This call does NOT
 * take them in that order: every weight is held OUTPUT-MAJOR, the [out][in] order of a
 * linear layer's weight matrix, i.e. the transposes [d_h][d] and [H][r][d].  Weights held
 * [d][d_h] / [d][H][r] must be transposed (made contiguous in the order below) first; passing
 * them untransposed is not detected and gives wrong rows.  The reason: the d weights that
 * produce one output coordinate are then contiguous, so both operands of the product are
 * read along d in 16-byte runs (the decode-step append reads each column's weights as one
 * run; held [d][out], a column's weights sit d rows apart).
 *   X        device, [n_rows][d]     in L->dtype
 *   W_SK     device, [d_h][d]        in L->dtype, element [c][k] = W_SK[k][c]
 *   W_SV     device, [d_h][d]        in L->dtype, element [c][k] = W_SV[k][c]
 *   U_K      device, [H][r][d]       in L->dtype, element [h][j][k] = U_K[h][k][j]
 *   U_V      device, [H][r][d]       in L->dtype, element [h][j][k] = U_V[h][k][j]
 *   row_req  device, [n_rows] int32  request of each row, 0 <= row_req[n] < (table rows)
 *   row_pos  device, [n_rows] int32  token position of each row; rows must address
 *                                    distinct (request, position) pairs
 *   page_table device, [*][max_pages_per_req] int32; the caller assigns the pages
 *   pool     device, num_pages * lrkv_page_bytes(L) bytes
 * Grouped layouts take one shared projection per group: W_SK and W_SV as [G][d_h][d].
 * d must be a positive multiple of 8.  n_rows == 0 is a no-op returning LRKV_OK. */
int lrkv_append(const lrkv_layout* L, const void* X, int32_t n_rows, int32_t d,
                const void* W_SK, const void* W_SV, const void* U_K, const void* U_V,
                const int32_t* row_req, const int32_t* row_pos, const int32_t* page_table,
                int32_t max_pages_per_req, void* pool, int64_t num_pages, void* stream);

/* Key-norm step of an append (LRKV notes §8, RMSNorm paragraph), for layouts with
 * key_norm = 1.  An RMSNorm of the key divides the full key k = S_K + R_K[h] B_K[h]^T by
 *   n_h = sqrt(|S_K + R_K[h] B_K[h]^T|^2 / d_h + eps),
 * a quantity of the full key that neither branch has alone (its square holds the cross
 * term 2 S_K B_K[h] R_K[h]^T).  For each appended row n and head h this reads the row's
 * stored S_K and R_K[h] (written by lrkv_append: enqueue this after it, on the same stream),
 * forms n_h with float32 accumulation and writes 1/n_h, rounded to nearest even in
 * L->dtype, at N[h][row_pos[n] % P] of the row's page; no other byte changes.  lrkv_decode
 * and lrkv_decode_rope then multiply each summed score by its key's stored 1/n_h.  A fixed
 * per-channel gain of the norm belongs on the query side (the caller's q).
 *   B_K        device, [H][d_h][r] in L->dtype
 *   eps        host value >= 0
 *   row_req, row_pos, page_table, max_pages_per_req, pool, num_pages: as in lrkv_append
 * bf16 layouts (16, 128, 56) and (32, 128, 32) with key_norm = 1; others return
 * LRKV_ERR_UNSUPPORTED (key_norm = 0: LRKV_ERR_INVALID_ARG).  n_rows == 0: no-op. */
int lrkv_key_norms(const lrkv_layout* L, const void* B_K, float eps, const int32_t* row_req,
                   const int32_t* row_pos, int32_t n_rows, const int32_t* page_table,
                   int32_t max_pages_per_req, void* pool, int64_t num_pages, void* stream);

/* Infrastructure of this library, not an operation of the method: the workspace bytes
 * lrkv_decode needs for these sizes (the split partial tuples).  0 for invalid arguments. */
size_t lrkv_decode_workspace_bytes(const lrkv_layout* L, int32_t batch, int32_t q_len,
                                   int32_t max_seq_len, int32_t chunk_tokens);

/* Algorithm 2 of LRKV notes §3 (every step but the output projection W_O), read
 * straight from the factored paged cache.
 *
 * For request b, query row i and head h, with T_b = seq_lens[b] cached tokens (the new
 * token already appended) and the query at position T_b - q_len + i:
 *   p        = q[b,i,h] B_K[h]                       formed once, float32   (eq 6)
 *   s_j      = (q[b,i,h] . S_K[j] + p . R_K[h,j]) / sqrt(d_h)   for visible j
 *   a        = one softmax over the visible positions j <= T_b - q_len + i   (§2)
 *   out[b,i,h] = a S_V + (a R_V[h]) B_V[h]^T         both branches, same weights (eq 7)
 * The divisor is sqrt(d_h), the full head width, never sqrt(r) (LRKV notes §2).  Masked
 * positions are excluded by selection, so unused page slots may hold any bytes (NaN
 * included).  A row that sees no position gets zeros.  Long histories are split into
 * chunks whose partial (max, exp-sum, shared acc, private acc) tuples are merged with the
 * rescaling rule of the fused blockwise paragraph of §3.  q_len = 1 is one decode step;
 * q_len = T_b is causal prefill over the cache.
 *
 *   q          device, [batch][q_len][H][d_h]  in L->dtype
 *   B_K, B_V   device, [H][d_h][r]             in L->dtype
 *   pool       device, factored pages (layout above)
 *   page_table device, [batch][max_pages_per_req] int32
 *   seq_lens   device, [batch] int32, 0 <= seq_lens[b] <= max_seq_len
 *   max_seq_len  host value >= every seq_lens[b], and <= max_pages_per_req * P
 *   chunk_tokens host value: 0 picks the split.  With q_len == 1 and 16 to 1024 requests
 *              the batch's pages (request after request, from the lengths on the device)
 *              are cut into equal ranges, one per split workgroup, whatever the lengths;
 *              otherwise chunks of batch * q_len * max_seq_len / 256 tokens (one wave of
 *              256 split workgroups, 64 to 2048 tokens).  Else a positive multiple of P up
 *              to 4096: chunks of that many tokens
 *   out        device, [batch][q_len][H][d_h]  in L->dtype
 *   workspace  device, >= lrkv_decode_workspace_bytes(L, batch, q_len, max_seq_len,
 *              chunk_tokens) bytes, 256-byte aligned; contents need not be initialised
 * Accumulation is float32 throughout. */
int lrkv_decode(const lrkv_layout* L, const void* q, int32_t batch, int32_t q_len,
                const void* B_K, const void* B_V, const void* pool, const int32_t* page_table,
                int32_t max_pages_per_req, const int32_t* seq_lens, int32_t max_seq_len,
                int32_t chunk_tokens, void* out, void* workspace, size_t workspace_bytes,
                void* stream);

/* Rotary decode: the exact path of LRKV notes §8 for a model whose keys and queries carry
 * rotary position encoding.  Same cache, same arguments and the same output as lrkv_decode,
 * but the key of head h at position j is the reconstructed key turned by the rotation D_j of
 * position j, and q holds the query already turned at its own position (q~):
 *   k_j      = (S_K[j] + R_K[h, j] B_K[h]^T) D_j
 *   s_j      = q~ . k_j / sqrt(d_h) = ((q~ D_j^T) . S_K[j] + ((q~ D_j^T) B_K[h]) . R_K[h, j]) / sqrt(d_h)
 *   out[b,i,h] = softmax over the visible j, applied to S_V + R_V[h] B_V[h]^T (values unturned)
 * The cache holds unrotated rows (lrkv_append as usual).  Because D_j depends on the key
 * position, the private query (q~ D_j^T) B_K[h] cannot be formed once (eq 6): this call forms,
 * per page and head, the private part of the unrotated keys P = R_K[h] B_K[h]^T on the matrix
 * cores (float32) and then, per feature pair m, a = k_2m q~_2m + k_2m+1 q~_2m+1 and
 * b = k_2m q~_2m+1 - k_2m+1 q~_2m of the unrotated key k, so that s_j sums c a + s b over the
 * pairs; it does more arithmetic than lrkv_decode.  The S_K part of a and b is exact; P
 * enters rounded to f16 (11 significant bits), so the entries of P and of q~ must stay below
 * 65504 (the largest finite f16) in magnitude, or the scores overflow.
 * D_j turns feature pairs (2m, 2m+1) of a row vector:
 *   (x_2m, x_2m+1) D_j = (x_2m c - x_2m+1 s,  x_2m s + x_2m+1 c),  (c, s) = rope_cs[j][m]
 *   rope_cs    device, float32 [rope_rows][d_h/2][2], (cos, sin) of position j in row j;
 *              rope_rows >= max_seq_len; 16-byte aligned
 *   workspace  >= lrkv_decode_rope_workspace_bytes(...) bytes, 256-byte aligned
 * Chunked split only (chunk_tokens 0 = automatic, else a multiple of P up to 4096), any
 * q_len.  bf16 variants only: (16, 128, 56) and (32, 128, 32); others return
 * LRKV_ERR_UNSUPPORTED. */
int lrkv_decode_rope(const lrkv_layout* L, const void* q, int32_t batch, int32_t q_len,
                     const void* B_K, const void* B_V, const void* pool,
                     const int32_t* page_table, int32_t max_pages_per_req,
                     const int32_t* seq_lens, int32_t max_seq_len, int32_t chunk_tokens,
                     const float* rope_cs, int32_t rope_rows, void* out, void* workspace,
                     size_t workspace_bytes, void* stream);

/* Infrastructure of this library: the workspace bytes lrkv_decode_rope needs. */
size_t lrkv_decode_rope_workspace_bytes(const lrkv_layout* L, int32_t batch, int32_t q_len,
                                        int32_t max_seq_len, int32_t chunk_tokens);

/* The private queries of eq 6 (LRKV notes §3: p_h = q_h B_K[h], one r-vector per query row
 * and head, shared by every key position) formed once per query row, for lrkv_decode_pq.
 * lrkv_decode forms them inside each of its split workgroups (each reads all of B_K); a
 * decode step can instead form them here (or with the step's new rows in one launch,
 * lrkv_append_pq: p depends on q and B_K only) and hand them to lrkv_decode_pq.
 *   q          device, [batch][q_len][H][d_h] in L->dtype (the decode call's queries)
 *   B_K        device, [H][d_h][r] in L->dtype
 *   p          device, >= lrkv_private_queries_bytes(L, batch, q_len) bytes, 16-byte
 *              aligned, written by this call.  Its layout is this library's (per row and
 *              head, float32 sums over d_h rounded to bfloat16 hi + lo pairs per 8-rank
 *              chunk for a bf16 cache, float32 for a float32 cache, with zero padding): it is
 *              only read by lrkv_decode_pq with the same layout, batch and q_len.
 * Every compiled layout: (4, 16, 4) float32; (16, 128, 56) and (32, 128, 32) bf16, with or
 * without key norms (which p does not involve); (32, 128, 32) bf16 in 2 groups (a row then
 * holds one block per group of 16 heads).  batch * q_len <= 4194304 rows
 * (LRKV_ERR_INVALID_ARG beyond).  Same arithmetic, in the same order, as lrkv_decode's own
 * formation, so lrkv_decode_pq's output equals lrkv_decode's bit for bit. */
int lrkv_private_queries(const lrkv_layout* L, const void* q, int32_t batch, int32_t q_len,
                         const void* B_K, void* p, size_t p_bytes, void* stream);

/* Infrastructure of this library: the bytes of lrkv_private_queries' output (0 for an
 * unsupported layout or invalid sizes). */
size_t lrkv_private_queries_bytes(const lrkv_layout* L, int32_t batch, int32_t q_len);

/* lrkv_append and lrkv_private_queries in one call: the n_rows new rows of Algorithm 1
 * (LRKV notes §3) appended to the pool, and the private queries of the batch * q_len query
 * rows q formed into p, with every argument of both checked before anything is launched
 * (arguments and their rules as in those two calls).  For 1..8 new rows of a bf16 cache
 * the two products run as one launch, the formation on compute units the few append
 * workgroups leave free (the decode step's case); otherwise as the two calls, in order, on
 * `stream`.  Layouts as lrkv_private_queries (a key-norm layout's norms are then written by
 * lrkv_key_norms, as after lrkv_append). */
int lrkv_append_pq(const lrkv_layout* L, const void* X, int32_t n_rows, int32_t d,
                   const void* W_SK, const void* W_SV, const void* U_K, const void* U_V,
                   const int32_t* row_req, const int32_t* row_pos, const int32_t* page_table,
                   int32_t max_pages_per_req, void* pool, int64_t num_pages, const void* q,
                   int32_t batch, int32_t q_len, const void* B_K, void* p, size_t p_bytes,
                   void* stream);

/* lrkv_decode with the private queries given (p from lrkv_private_queries for these q,
 * B_K, batch and q_len) instead of B_K: the same split and merge, the same output bit for
 * bit, without each split workgroup reading B_K and forming p.  Arguments as lrkv_decode,
 * with p and its size p_bytes in place of B_K: p_bytes <
 * lrkv_private_queries_bytes(L, batch, q_len), like a workspace smaller than
 * lrkv_decode_workspace_bytes(L, batch, q_len, max_seq_len, chunk_tokens), returns
 * LRKV_ERR_INVALID_ARG before anything is launched.  Layouts as lrkv_private_queries; a call of q_len >= 64 over
 * a one-group bf16 layout without key norms (which lrkv_decode sends to its multi-query
 * kernel) returns LRKV_ERR_UNSUPPORTED. */
int lrkv_decode_pq(const lrkv_layout* L, const void* q, const void* p, size_t p_bytes,
                   int32_t batch, int32_t q_len, const void* B_V, const void* pool, const int32_t* page_table,
                   int32_t max_pages_per_req, const int32_t* seq_lens, int32_t max_seq_len,
                   int32_t chunk_tokens, void* out, void* workspace, size_t workspace_bytes,
                   void* stream);

/* lrkv_decode without a workspace argument, for callers that cannot allocate device memory
 * for it (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, semantics and kernels as lrkv_decode, minus workspace and
 * workspace_bytes: the split partials go to a fixed scratch array of 16 MiB (16,777,216
 * bytes) compiled into the library, one per GPU, held by each GPU the library runs on until
 * the process ends.  Nothing is allocated or freed by this call.
 *  - A call whose lrkv_decode_workspace_bytes(...) exceeds 16 MiB returns LRKV_ERR_SCRATCH
 *    before touching the device (at B=8, T=4096 with the automatic split: 3 MiB).
 *  - Every call on one GPU uses that GPU's one array, which keeps the last call's contents
 *    (nothing in it needs to start at any value).  Calls that may overlap on one GPU (other
 *    streams, other host threads) race on it and must be ordered by the caller.
 *  - The first call on a GPU looks up the array's device address on that GPU (the device
 *    of `stream`, else the current device) and keeps it for the process. */
int lrkv_decode_noalloc(const lrkv_layout* L, const void* q, int32_t batch, int32_t q_len,
                        const void* B_K, const void* B_V, const void* pool,
                        const int32_t* page_table, int32_t max_pages_per_req,
                        const int32_t* seq_lens, int32_t max_seq_len, int32_t chunk_tokens,
                        void* out, void* stream);

/* Counts the device-side index values that lrkv_append and lrkv_decode trust without
 * checking them (they read them on the device; a check there would need a
 * synchronization).  For callers who want to validate their tables first, for example in
 * a debug run: enqueue this on the same stream before the calls it guards.  The rules
 * are those of the page layout above (LRKV notes §3, one page table for shared and
 * private rows):
 *   lengths  (if seq_lens != NULL)  0 <= seq_lens[b] <= max_seq_len, for b < batch
 *   pages    (if seq_lens != NULL)  for each b with a valid length and each page index
 *            p < ceil(seq_lens[b] / P): 0 <= page_table[b * max_pages_per_req + p] < num_pages
 *   rows     (if row_req != NULL)   0 <= row_req[n] < batch, 0 <= row_pos[n] <
 *            max_pages_per_req * P, and the page holding (row_req[n], row_pos[n]) is in
 *            [0, num_pages), for n < n_rows
 * Distinctness of the appended (request, position) pairs is not checked.
 *   page_table device, [batch][max_pages_per_req] int32
 *   seq_lens   device, [batch] int32, or NULL
 *   row_req, row_pos  device, [n_rows] int32 each, or both NULL
 *   errors     device, one int32, written asynchronously on `stream`: the number of
 *              violations found (0: every checked value is valid).  Device pointers need
 *              4-byte alignment here.
 * Returns LRKV_OK once the check is enqueued (two small kernels; nothing allocated), or
 * LRKV_ERR_INVALID_ARG for host-side argument errors (batch, max_pages_per_req or
 * num_pages <= 0, max_seq_len outside [0, max_pages_per_req * P], a NULL page_table or
 * errors, one of row_req / row_pos NULL without the other). */
int lrkv_check_indices(const lrkv_layout* L, const int32_t* page_table, int32_t batch,
                       int32_t max_pages_per_req, const int32_t* seq_lens, int32_t max_seq_len,
                       const int32_t* row_req, const int32_t* row_pos, int32_t n_rows,
                       int64_t num_pages, int32_t* errors, void* stream);

/* ---------------------------------------------------------------------------------------
 * Shared-prefix page reuse and reclamation (LRKV notes §3, the note after Algorithm 1:
 * shared and private pages must keep the same token numbering and reclamation lifetime, or
 * reusing a prefix or releasing a request can leave the two paths of one position pointing
 * at different histories).  One page id holds every section of its tokens, so a page shared,
 * copied or freed moves its shared rows, private rows (and key-norm reciprocals) together.
 *
 * The allocator is host code over caller-owned host arrays; it keeps no other state.  It is
 * not thread-safe: one caller at a time per lrkv_page_pool. */
typedef struct lrkv_page_pool {
  int64_t num_pages;   /* pages of the pool */
  int64_t num_free;    /* free page ids on the stack */
  int32_t* refcount;   /* host, [num_pages]: requests holding each page (0: free) */
  int32_t* free_stack; /* host, [num_pages]: free ids; the next allocation takes
                          free_stack[num_free - 1] */
} lrkv_page_pool;

/* Every page free; allocations then return ids 0, 1, 2, ... in order. */
int lrkv_pages_init(lrkv_page_pool* pp, int32_t* refcount, int32_t* free_stack,
                    int64_t num_pages);
/* Takes n free pages (reference count 1) into ids[0..n); LRKV_ERR_NO_PAGES, with nothing
 * taken, if fewer than n are free. */
int lrkv_pages_alloc(lrkv_page_pool* pp, int32_t n, int32_t* ids);
/* One more reference to each listed page (a request that shares it); every page must be in
 * use, else LRKV_ERR_INVALID_ARG and nothing changes. */
int lrkv_pages_retain(lrkv_page_pool* pp, const int32_t* ids, int32_t n);
/* Drops one reference per listed page (an id listed twice drops two); pages left with none
 * return to the free stack in list order.  A page with fewer references than listings:
 * LRKV_ERR_INVALID_ARG and nothing changes. */
int lrkv_pages_release(lrkv_page_pool* pp, const int32_t* ids, int32_t n);
/* A new request that continues the first prefix_len tokens of another (shared prefix):
 * child_row[k] = parent_row[k] for the prefix_len / P full pages (one more reference each,
 * never written again: later tokens go to later pages); if prefix_len % P != 0 the page
 * holding the prefix's last tokens is copied, every section of it, into a newly allocated
 * page (enqueued on `stream`), which becomes the child's, so both requests can append past
 * the prefix without touching each other's rows.  Host rows, device pool; child_row
 * entries past the prefix are not written.  LRKV_ERR_NO_PAGES if the copy has no page. */
int lrkv_fork_prefix(const lrkv_layout* L, lrkv_page_pool* pp, const int32_t* parent_row,
                     int32_t prefix_len, int32_t* child_row, int32_t max_pages_per_req,
                     void* pool, void* stream);
/* Copies whole pages (every section) src_ids[i] -> dst_ids[i], i < n, on the device.
 * src_ids, dst_ids: device int32 [n]; pool: device, 16-byte aligned. */
int lrkv_copy_pages(const lrkv_layout* L, void* pool, const int32_t* src_ids,
                    const int32_t* dst_ids, int32_t n, void* stream);

/* Infrastructure of this library (measurement), not an operation of the method: a plain
 * streaming read of `bytes` bytes of device memory at `buf` by `workgroups` workgroups of
 * 256 threads (16-byte loads), the bound for any kernel that must read those bytes once.
 *   buf   device, 16-byte aligned, bytes > 0 a multiple of 16
 *   sink  device, workgroups * 16 bytes, 16-byte aligned: each workgroup writes the XOR
 *         fold of what it read (written so that no read can be elided)
 * Enqueued on `stream`; LRKV_ERR_INVALID_ARG for bad arguments, LRKV_ERR_HIP if the launch
 * fails. */
int lrkv_read_probe(const void* buf, uint64_t bytes, int32_t workgroups, void* sink,
                    void* stream);

/* Infrastructure of this library, not an operation of the method: the text of a status
 * code (static storage). */
const char* lrkv_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* LRKV_H */
