/*
 * attn_decode.h -- C ABI of the MI355X (gfx950) decode-attention library.
 *
 * One call computes one decode step of attention for one layer: a single new
 * query token per sequence attends to that sequence's KV cache,
 *
 *     out[b,h] = softmax(scale * q[b,h] . K[b,g(h)]^T + M) . V[b,g(h)]
 *
 * (attention equation, xuesongtap.github.io "attention-head" note, section 1).
 * The layout of the cache follows from head sharing: [B, H_kv, T, d] with
 * H_kv == H_q (MHA), 1 < H_kv < H_q (GQA) or H_kv == 1 (MQA); query head h
 * reads KV head g(h) = floor(h / (H_q / H_kv)) -- equal, contiguously
 * numbered groups (attention-head sections 2, 2.1, 2.2; the toolsku article's
 * GQA module expands KV heads the same way).  MLA reads a latent cache
 * [B, T, d_c + d_rope] with the key up-projection absorbed into the query and
 * the value up-projection left to the caller (attention-head sections
 * 5.2-5.3).
 *
 * Conventions shared by every entry point:
 *  - Pointers named q, k, v, latent, out, lse_out, seq_lens, ring_head,
 *    o_part, lse_part and workspace are DEVICE pointers owned by the caller.
 *    The library never allocates, frees or synchronises; every call only
 *    enqueues kernels on `stream` (a hipStream_t; NULL = the null stream) and
 *    returns.  The caller keeps inputs alive and unmodified until the stream
 *    reaches the work.  Calls are thread-safe; the only global state is the
 *    per-GPU device array of attn_decode_gqa_noalloc (see there).
 *  - Tensors are dense, row-major, in exactly the shapes given.  q, k, v,
 *    latent and workspace must be 16-byte aligned; out, lse_out and the
 *    partial buffers 4-byte aligned.
 *  - Sequence b's cache holds T_b = seq_lens[b] tokens including the current
 *    one; the query is position t = T_b - 1 and full causal attention sees
 *    positions 0..t (attention-head section 5.3, single-token causal decode
 *    over the valid cached tokens).  seq_lens == NULL means T_b = T_cap.
 *  - Masked positions drop out of the softmax (M = -inf), visible ones add 0.
 *    Masked cache rows are never read: the kernels load only the visible
 *    range (attention-head section 3: a window pays off only when the kernel
 *    skips masked positions).
 *  - Results are float32.  lse_out (nullable) receives the natural-log
 *    log-sum-exp of the scaled visible scores.  A query with no visible key
 *    gets out = 0 and lse = -inf.
 *  - All argument checks use host values only and happen before any HIP
 *    call; a failing check returns its code and enqueues nothing.  Values
 *    inside device arrays are not checked on the host; see each function for
 *    how out-of-range values are treated.
 */
#ifndef ATTN_DECODE_H
#define ATTN_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q / k / v.  Accumulation is always float32. */
typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype;

/* Status codes returned by every int-returning entry point. */
enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = -1,        /* a required pointer is NULL                     */
  ATTN_ERR_SHAPE = -2,       /* H <= 0, T_cap <= 0, B < 0, H_q % H_kv != 0     */
  ATTN_ERR_DTYPE = -3,       /* dtype not an attn_dtype value                  */
  ATTN_ERR_UNSUPPORTED = -4, /* head dim / latent widths / dtype combo absent  */
  ATTN_ERR_WINDOW = -5,      /* window < 0, or ring mode with window > T_cap   */
  ATTN_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than required        */
  ATTN_ERR_ALIGN = -7,       /* a pointer misses its alignment                 */
  ATTN_ERR_HIP = -8,         /* the HIP runtime reported an error on launch    */
  ATTN_ERR_ARG = -9          /* bad scalar: scale not finite, num_splits range */
};

/* Largest accepted num_splits. */
#define ATTN_MAX_SPLITS 1024

/*
 * attn_decode_gqa -- one decode step of MHA / GQA / MQA attention.
 *
 *   q         [B, H_q, d]           dtype
 *   k, v      [B, H_kv, T_cap, d]   dtype   (row (b, g, slot) is d contiguous
 *                                            elements: attention-head section 2
 *                                            layout [batch, head, seq, dim])
 *   out       [B, H_q, d]           float32
 *   lse_out   [B, H_q]              float32, may be NULL
 *   seq_lens  [B] int32 logical lengths T_b, may be NULL (all T_cap).
 *             Linear mode: values are clamped to [0, T_cap].
 *             Ring mode: any value >= 0 (the ring keeps the newest T_cap);
 *             negative values are treated as 0.
 *   ring_head [B] int32, may be NULL.  Non-NULL selects ring-buffer
 *             addressing (attention-head section 3: a pure sliding-window
 *             layer may reuse out-of-window slots as a ring): the cache has
 *             T_cap slots, ring_head[b] is the slot holding the newest
 *             position t, and position j sits in slot
 *             (ring_head[b] - (t - j)) mod T_cap.  Only the last T_cap
 *             positions are resident.  Values are reduced mod T_cap.
 *   B, H_q, H_kv, T_cap, d   shapes; d in {64, 128, 256}; H_q % H_kv == 0;
 *             B == 0 is a no-op (pointers may then be NULL).
 *   dtype     ATTN_F32 or ATTN_BF16 (all of q, k, v).
 *   window    0: no window (in ring mode: every resident position).
 *             w > 0: the query at t sees t-w+1 .. t (attention-head section
 *             3, worked example w = 3: row 8 sees 6, 7, 8).  Ring mode
 *             requires w <= T_cap.
 *   scale     softmax scale; <= 0 or NaN selects 1/sqrt(d) (section 1).
 *   num_splits  number of pieces the visible range of a sequence is cut into
 *             (their results are merged by attn_combine's rule);
 *             0 = chosen by the library (attn_decode_gqa_splits tells which).
 *   workspace, workspace_bytes  scratch for split results; required when the
 *             split count is > 1, size from attn_decode_gqa_workspace_bytes.
 *             Contents on entry are ignored.  When the library picks the
 *             splits and the batch has fewer (sequence, KV head) units than
 *             work groups, a call with seq_lens assigns pieces by visible
 *             length instead (attn_gqa_plan.balanced_groups, and
 *             .even_split for how); a workspace smaller than that size but
 *             large enough for the fixed splits runs the fixed splits.
 *   stream    hipStream_t.
 */
int attn_decode_gqa(const void* q, const void* k, const void* v, float* out,
                    float* lse_out, const int32_t* seq_lens,
                    const int32_t* ring_head, int B, int H_q, int H_kv,
                    int T_cap, int d, int dtype, int window, float scale,
                    int num_splits, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Bytes of the device array attn_decode_gqa_noalloc keeps its split results
 * in (16 MiB per GPU). */
#define ATTN_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * attn_decode_gqa_noalloc -- attn_decode_gqa for callers that cannot
 * allocate device memory or manage a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.
 *
 * Same arguments, meaning and result as attn_decode_gqa without workspace /
 * workspace_bytes: the split partials (and the balanced list's parts) go to
 * a device array of ATTN_NOALLOC_SCRATCH_BYTES that the library holds on
 * each GPU it runs on until the process ends.  The call allocates nothing
 * (no hipMalloc or hipFree, no allocating library routine); its first call
 * on a device looks up that device's array address once.  The caller still
 * passes inputs and outputs.
 *   - A plan whose fixed splits need more than ATTN_NOALLOC_SCRATCH_BYTES
 *     (attn_decode_gqa_workspace_bytes with ring and num_splits as given,
 *     for the fixed part) returns ATTN_ERR_WORKSPACE before any HIP call;
 *     the balanced list is used only when it fits.
 *   - Every call on one GPU shares that GPU's array: calls that overlap on
 *     one GPU (two streams, or two threads each with its own stream) race
 *     and give unspecified results.  Calls ordered on one stream are safe.
 *     The array's contents on entry are never read before they are written.
 */
int attn_decode_gqa_noalloc(const void* q, const void* k, const void* v,
                            float* out, float* lse_out, const int32_t* seq_lens,
                            const int32_t* ring_head, int B, int H_q, int H_kv,
                            int T_cap, int d, int dtype, int window, float scale,
                            int num_splits, void* stream);

/* Split count attn_decode_gqa would use for these arguments (>= 1), or a
 * negative status if the shape arguments are invalid. */
int attn_decode_gqa_splits(int B, int H_q, int H_kv, int T_cap, int d,
                           int dtype, int window, int ring, int num_splits);

/* Workspace bytes attn_decode_gqa needs for these arguments (0 when no
 * workspace is needed, (size_t)-1 when the arguments are invalid). */
size_t attn_decode_gqa_workspace_bytes(int B, int H_q, int H_kv, int T_cap,
                                       int d, int dtype, int window, int ring,
                                       int num_splits);

/* How attn_decode_gqa and its _global / _paged / _multi forms would run a
 * call: which kernel, how the visible range is split, the launch shape and
 * the workspace it needs.  The library fills the whole struct as declared
 * here: a caller must use this header with the library built from it (new
 * fields are added at the end). */
typedef struct {
  int kernel;          /* 0 = vector-ALU kernel, 1 = matrix-core kernel      */
  int splits;          /* pieces of each visible range (1 = no combine pass) */
  int chunk;           /* positions per piece                                */
  int heads_per_item;  /* (head, token) columns one work group serves        */
  int tile_rows;       /* positions per wave per tile                        */
  int waves;           /* waves per work group                               */
  long long groups;    /* work groups of the decode kernel                   */
  size_t workspace_bytes; /* workspace the call needs (0: none)              */
  int balanced_groups; /* > 0: a call that passes seq_lens (with out 16-byte
                        * aligned and this workspace) cuts the visible rows
                        * by their lengths over at most this many work
                        * groups instead of `splits` fixed pieces; 0: never
                        * (also for rings, whose visible ranges are alike)  */
  int even_split;      /* with balanced_groups > 0: 1 = every work group
                        * takes the same number of 32-row tiles of the
                        * batch's rows laid end to end (a group may finish
                        * one sequence and start the next: matrix-core
                        * kernel, d <= 128); 0 = each sequence is cut into
                        * pieces of one common size, at least one per
                        * sequence                                         */
} attn_gqa_plan;

/* Fills *plan for these arguments: q_len query tokens per sequence (1 for
 * decode), n_global as for attn_decode_gqa_global (0 otherwise); a paged call
 * plans as T_cap = max_pages * page_size with ring = 0.  Returns ATTN_OK or
 * the status the call would return for these arguments; plan must not be
 * NULL (ATTN_ERR_NULL). */
int attn_decode_gqa_plan(int B, int q_len, int H_q, int H_kv, int T_cap, int d,
                         int dtype, int window, int ring, int n_global,
                         int num_splits, attn_gqa_plan* plan);

/* Largest accepted q_len (query tokens per sequence). */
#define ATTN_MAX_QLEN 1024

/*
 * attn_decode_gqa_multi -- q_len query tokens per sequence in one call
 * (speculative-decode verification, chunked prefill).  The tokens are the
 * last q_len positions of each cache, already written: token l sits at
 * t_l = T_b - q_len + l and sees exactly what a single decode query at t_l
 * sees (positions 0..t_l -- causal inside the chunk -- cut to its own
 * window t_l-w+1..t_l; in ring mode only positions still resident after
 * the whole chunk).  A token with t_l < 0 sees nothing (out 0, lse -inf).
 *
 *   q        [B, q_len, H_q, d]  dtype (token-major)
 *   out      [B, q_len, H_q, d]  float32
 *   lse_out  [B, q_len, H_q]     float32, may be NULL
 *   q_len    1..ATTN_MAX_QLEN; 1 is attn_decode_gqa.
 *   ring mode requires window + q_len - 1 <= T_cap (the first token's
 *   window must be resident), else ATTN_ERR_WINDOW.
 *   Everything else as for attn_decode_gqa; the workspace size comes from
 *   attn_decode_gqa_plan (q_len as given).
 * Each (head, token) pair is a column of its KV head's group: the group's
 * K/V rows are read once for all q_len * H_q / H_kv columns.
 */
int attn_decode_gqa_multi(const void* q, const void* k, const void* v,
                          float* out, float* lse_out, const int32_t* seq_lens,
                          const int32_t* ring_head, int B, int q_len, int H_q,
                          int H_kv, int T_cap, int d, int dtype, int window,
                          float scale, int num_splits, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Largest accepted n_global. */
#define ATTN_MAX_GLOBAL 65536

/*
 * attn_decode_gqa_global -- attn_decode_gqa over a linear cache with a
 * sliding window plus global positions (attention-head section 3, the
 * window-plus-global pattern, example G = {0, 5}).
 *
 *   global_pos [n_global] int32 device array: the global positions G,
 *             sorted ascending, no repeats, each in [0, T_cap).  Shared by
 *             the whole batch.
 *   n_global  0..ATTN_MAX_GLOBAL; 0 (global_pos may then be NULL) gives
 *             exactly attn_decode_gqa without ring.
 *   The query at t = T_b - 1 sees its window t-w+1 .. t plus every g in G
 *   with g < t-w+1; a query that is itself in G (t in G) sees all of 0..t.
 *   window == 0 means no window (G then changes nothing).
 *   Every other argument, and the split / workspace rules, as for
 *   attn_decode_gqa with ring_head == NULL; size the workspace with
 *   attn_decode_gqa_global_workspace_bytes.
 *   Values of global_pos are not checked on the host.  An unsorted list or
 *   one with repeats gives an unspecified result; entries outside
 *   [0, T_cap) are clamped to a cache row, so no access leaves the cache.
 */
int attn_decode_gqa_global(const void* q, const void* k, const void* v,
                           float* out, float* lse_out, const int32_t* seq_lens,
                           const int32_t* global_pos, int n_global, int B,
                           int H_q, int H_kv, int T_cap, int d, int dtype,
                           int window, float scale, int num_splits,
                           void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * attn_decode_gqa_paged -- attn_decode_gqa over a paged KV cache (the KV
 * cache paging that the baidu article, section 四.3, names as the serving
 * side of MQA / GQA and MLA; the pages fix no layout, this one is the
 * library's).
 *
 *   k_pages, v_pages [num_pages, H_kv, page_size, d] dtype: a pool of
 *             pages; page p holds page_size consecutive positions of one
 *             sequence for every KV head, each head's rows contiguous.
 *   block_table [B, max_pages] int32: position j of sequence b lives in
 *             page block_table[b][j / page_size], row j % page_size.
 *             Only entries 0 .. (T_b - 1) / page_size of a row are read.
 *   seq_lens  [B] int32, may be NULL (all max_pages * page_size); clamped
 *             to [0, max_pages * page_size].
 *   page_size a power of two, 16 .. 65536 (else ATTN_ERR_UNSUPPORTED).
 *   num_pages >= 1, max_pages >= 1; max_pages * page_size <= 2^30 and
 *             num_pages * H_kv * page_size < 2^31 (else ATTN_ERR_SHAPE).
 *   window    as for attn_decode_gqa (no ring mode on a paged cache).
 *   q_len     query tokens per sequence, as for attn_decode_gqa_multi (q,
 *             out and lse_out then have its token-major shapes); 1 = decode.
 *   Everything else as for attn_decode_gqa.  Split count and workspace are
 *   those of attn_decode_gqa_plan with T_cap = max_pages * page_size and
 *   ring = 0 (for q_len = 1 also attn_decode_gqa_splits / _workspace_bytes).
 *   Table entries are not checked on the host: ids outside [0, num_pages)
 *   are clamped to the pool, so no access leaves it (the result is then
 *   unspecified).
 */
int attn_decode_gqa_paged(const void* q, const void* k_pages,
                          const void* v_pages, float* out, float* lse_out,
                          const int32_t* seq_lens, const int32_t* block_table,
                          int max_pages, int B, int q_len, int H_q, int H_kv,
                          int num_pages, int page_size, int d, int dtype,
                          int window, float scale, int num_splits,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Split count and workspace bytes of attn_decode_gqa_global, with the same
 * return conventions as attn_decode_gqa_splits / _workspace_bytes. */
int attn_decode_gqa_global_splits(int B, int H_q, int H_kv, int T_cap, int d,
                                  int dtype, int window, int n_global,
                                  int num_splits);
size_t attn_decode_gqa_global_workspace_bytes(int B, int H_q, int H_kv,
                                              int T_cap, int d, int dtype,
                                              int window, int n_global,
                                              int num_splits);

/*
 * attn_decode_mla -- one decode step of absorbed multi-head latent attention.
 *
 *   q       [B, H, d_c + d_rope]  bf16: each row is [q~ | q^R], the content
 *           query already multiplied by the head's key up-projection
 *           transposed (attention-head section 5.2), followed by the RoPE
 *           query (section 5.3).
 *   latent  [B, T_cap, d_c + d_rope]  bf16: each row is [c_j | k^R_j], the
 *           normalised latent followed by the shared RoPE key (the one-tensor
 *           cache [batch, seq, compressed_kv_dim + rope_dim] of the baidu
 *           article, section 二).
 *   out     [B, H, d_c] float32, 16-byte aligned: z = sum_j p_j c_j, the
 *           latent-space result before the value up-projection
 *           (attention-head section 5.2).
 *   lse_out [B, H] float32, may be NULL.
 *   seq_lens [B] int32, may be NULL (all T_cap); clamped to [0, T_cap].
 *   Scores are scale * (q~ . c_j + q^R . k^R_j): one dot product over the
 *   whole row, one softmax over the sum (section 5.3).
 *   (d_c, d_rope) = (512, 64) and (256, 64) are supported (the latter is the
 *   32-head, latent-256 geometry of the attention-head note's section 6 model
 *   table; any H works).
 *   scale   must be > 0 and finite: 1/sqrt(d_head_content + d_rope) with the
 *           model's per-head content width (section 5.3 keeps that
 *           denominator; the latent width r does not enter it).
 *   Precision, (512, 64): the value product runs on the matrix cores in
 *   fp16: every bf16 latent value with 2^-14 <= |x| <= 65504 converts
 *   exactly (smaller ones with an absolute error below 2^-25); entries
 *   beyond 65504 overflow and are outside the accepted range.  The scores
 *   are exact bf16 products on fixed splits; with lengths that take the
 *   balanced work list they are formed in fp16 too, under the same range
 *   condition on q.  The softmax weights enter the value product rounded to
 *   fp16 (11 significant bits); accumulation is float32; when the call
 *   splits, each piece's normalised partial value (a weighted mean of latent
 *   values, so inside the same range) is stored in fp16 before the merge.
 *   (256, 64): q and
 *   the latent stay bf16 (exact products), the weights carry about 16
 *   significant bits (a bf16 high part plus a bf16 remainder), partials are
 *   float32.
 *   num_splits / workspace / stream as for attn_decode_gqa, with
 *   attn_decode_mla_workspace_bytes giving the size.
 */
int attn_decode_mla(const void* q, const void* latent, float* out,
                    float* lse_out, const int32_t* seq_lens, int B, int H,
                    int T_cap, int d_c, int d_rope, float scale,
                    int num_splits, void* workspace, size_t workspace_bytes,
                    void* stream);

int attn_decode_mla_splits(int B, int H, int T_cap, int d_c, int d_rope,
                           int num_splits);

size_t attn_decode_mla_workspace_bytes(int B, int H, int T_cap, int d_c,
                                       int d_rope, int num_splits);

/*
 * attn_decode_mla_paged -- attn_decode_mla over a paged latent cache (the
 * paging strategy the baidu article, section 四.3, says an MLA stack must
 * adapt; the layout is the library's).
 *
 *   latent_pages [num_pages, page_size, d_c + d_rope] bf16: a pool of
 *             pages of page_size consecutive latent rows [c_j | k^R_j].
 *   block_table [B, max_pages] int32: position j of sequence b lives in
 *             page block_table[b][j / page_size], row j % page_size; only
 *             entries 0 .. (T_b - 1) / page_size are read.
 *   seq_lens  [B] int32, may be NULL (all max_pages * page_size); clamped
 *             to [0, max_pages * page_size].
 *   page_size, num_pages, max_pages: as for attn_decode_gqa_paged (with
 *             H_kv = 1 in the pool-size bound).
 *   q_len     query tokens per sequence as for attn_decode_mla_multi (its
 *             q / out / lse_out shapes); 1 = decode.
 *   Everything else as for attn_decode_mla; split count and workspace are
 *   those of attn_decode_mla_splits / _workspace_bytes with
 *   T_cap = max_pages * page_size and H * q_len in place of H.  Table ids outside [0, num_pages) are
 *   clamped to the pool.
 */
int attn_decode_mla_paged(const void* q, const void* latent_pages, float* out,
                          float* lse_out, const int32_t* seq_lens,
                          const int32_t* block_table, int max_pages, int B,
                          int q_len, int H, int num_pages, int page_size,
                          int d_c, int d_rope, float scale, int num_splits,
                          void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * attn_decode_mla_multi -- attn_decode_mla with q_len query tokens per
 * sequence (the last q_len positions of the cache, already written; token l
 * at t_l = T_b - q_len + l sees positions 0..t_l, as in
 * attn_decode_gqa_multi).
 *
 *   q        [B, q_len, H, d_c + d_rope] bf16 (token-major)
 *   out      [B, q_len, H, d_c] float32, 16-byte aligned
 *   lse_out  [B, q_len, H] float32, may be NULL
 *   q_len    1..ATTN_MAX_QLEN.
 *   Everything else as for attn_decode_mla; split count and workspace are
 *   those of attn_decode_mla_splits / _workspace_bytes with H * q_len in
 *   place of H.  Every latent row is read once for all H * q_len columns.
 */
int attn_decode_mla_multi(const void* q, const void* latent, float* out,
                          float* lse_out, const int32_t* seq_lens, int B,
                          int q_len, int H, int T_cap, int d_c, int d_rope,
                          float scale, int num_splits, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * attn_combine -- merge results computed over S disjoint parts of each key
 * set.  With L = max_s lse_part[s] and w_s = exp(lse_part[s] - L):
 *     out = sum_s w_s o_part[s] / sum_s w_s,   lse = L + ln(sum_s w_s).
 * This is the softmax of the attention equation (attention-head section 1)
 * taken over a union of disjoint key sets.  Parts with lse = -inf are empty
 * and their o_part rows are not used; if all are, out = 0 and lse = -inf.
 *
 *   o_part   [B, H, S, d_v] float32     lse_part [B, H, S] float32
 *   out      [B, H, d_v]    float32     lse_out  [B, H] float32, may be NULL
 *   S in 1..ATTN_MAX_SPLITS, d_v in 1..4096; B == 0 is a no-op.
 */
int attn_combine(const float* o_part, const float* lse_part, float* out,
                 float* lse_out, int B, int H, int S, int d_v, void* stream);

/*
 * attn_kv_append -- write the current token's rows into a linear cache (the
 * step before a decode call: the pages' modules concatenate the new key and
 * value onto the cached ones along the sequence axis -- toolsku MHA / GQA /
 * MLA modules).  For every sequence b and head g:
 *     k_cache[b, g, positions[b], :] = k_new[b, g, :]   (and v likewise)
 *   k_cache, v_cache [B, H, T_cap, d]; k_new, v_new [B, H, d]; dtype as for
 *   attn_decode_gqa.  v_cache and v_new may both be NULL (one tensor only,
 *   e.g. an MLA latent cache [B, T_cap, d_c + d_rope] with H = 1).
 *   positions [B] int32: usually the length before the append (T_b - 1
 *   after it).  Positions outside [0, T_cap) are skipped.
 *   Rows must be a multiple of 16 bytes; pointers 16-byte aligned.
 */
int attn_kv_append(void* k_cache, void* v_cache, const void* k_new,
                   const void* v_new, const int32_t* positions, int B, int H,
                   int T_cap, int d, int dtype, void* stream);

/*
 * attn_kv_append_ring -- the ring-buffer form (attention-head section 3:
 * slots of positions that left the window are reused).  For every b the row
 * goes to slot (ring_head[b] + 1) mod T_cap, which then becomes the newest
 * slot: ring_head[b] is updated in place (device memory), ready for
 * attn_decode_gqa's ring mode.  An empty ring starts with ring_head =
 * T_cap - 1 so the first row lands in slot 0.  Other arguments as
 * attn_kv_append.
 */
int attn_kv_append_ring(void* k_cache, void* v_cache, const void* k_new,
                        const void* v_new, int32_t* ring_head, int B, int H,
                        int T_cap, int d, int dtype, void* stream);

/*
 * attn_kv_append_paged -- attn_kv_append into a paged pool (the layout of
 * attn_decode_gqa_paged; a latent pool [num_pages, page_size, d_c + d_rope]
 * is the case H = 1).  For every sequence b with
 * 0 <= positions[b] < max_pages * page_size and every head h:
 *     k_pages[block_table[b][pos / page_size], h, pos % page_size, :] = k_new[b, h, :]
 *   k_pages, v_pages [num_pages, H, page_size, d]; k_new, v_new [B, H, d];
 *   v_pages / v_new may both be NULL.  positions and block_table are device
 *   int32 arrays ([B] and [B, max_pages]); page ids outside [0, num_pages)
 *   are clamped to the pool.  Page geometry is checked as for
 *   attn_decode_gqa_paged; rows must be a multiple of 16 bytes.
 */
int attn_kv_append_paged(void* k_pages, void* v_pages, const void* k_new,
                         const void* v_new, const int32_t* positions,
                         const int32_t* block_table, int max_pages, int B, int H,
                         int num_pages, int page_size, int d, int dtype,
                         void* stream);

/* Bytes of the split buffers for S splits: o_part [B,H,S,d_v] and lse_part
 * [B,H,S], float32, each 256-byte aligned inside the workspace (0 if S<=1). */
size_t attn_decode_workspace_bytes(int B, int H, int d_v, int num_splits);

/* Static, human-readable text for a status code. */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_DECODE_H */
