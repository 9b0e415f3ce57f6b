/*
 * tilemix.h — C ABI of libtilemix.so: routed FP16/INT8 causal prefill attention
 * for AMD Instinct MI355X (gfx950).
 *
 * Sources cited below:
 *   [PL §n]  paperlayer.ai summary of arXiv 2608.17336, "TileMix: Tile-Centric
 *            Mixed-Precision Attention for LLM Inference Acceleration", section n
 *            (App. B/C/D = its appendix bullets).
 *   [AN]     ainews.surl.tw, "TileMix Mixes FP16 and INT8 Within the Attention
 *            Matrix, Reaching 2.22x FlashAttention Throughput for 4K Prefill on A100".
 *   [GS]     gist.science technical summary, "Resumen Tecnico", subsection on
 *            compact bitmask routing.
 *   [AF]     ai-feeds.com summary (Chinese), sections on interfaces to existing products
 *            and on limitations.
 *
 * Conventions shared by every call:
 *   - Every pointer argument is a DEVICE pointer unless marked "host".
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL = the null stream).  Nothing is synchronised and nothing allocated:
 *     the caller owns every buffer, including the attention workspace.
 *   - Tokens of all sequences are packed without padding, token-major:
 *     x[t][h][c] with t in [0, N), N = cu_seqlens[batch].  `cu_seqlens` is int32
 *     [batch+1] prefix sums of sequence lengths, cu_seqlens[0] = 0, non-
 *     decreasing, every length <= max_seqlen.  A fixed-length batch is
 *     cu_seqlens = {0, L, 2L, ...}.
 *   - Score tiles are 64 x 64 (query tile m, key tile n); T = ceil(max_seqlen/64).
 *   - Chunked prefill / decode (optional key prefix sums `cu_seqlens_k` with
 *     `max_seqlen_k` > 0): sequence b has Lq_b = cu_seqlens[b+1] - cu_seqlens[b]
 *     queries and Lk_b >= Lq_b keys, and its queries are the last Lq_b of its Lk_b
 *     positions (bottom-right causal alignment): key j is legal for query i iff
 *     j <= (Lk_b - Lq_b) + i.  Query tiles count from the first query, key tiles
 *     from the first key, Tk = ceil(max_seqlen_k/64).  Without cu_seqlens_k
 *     (max_seqlen_k = 0) the keys are the queries' own positions (prefill, Tk = T).
 *   - Arguments are validated on the host before any launch.  On failure a
 *     status other than TILEMIX_OK is returned, nothing is launched and
 *     tilemix_last_error() describes the problem.  A failed HIP launch returns
 *     TILEMIX_ERR_HIP.  Device-side contents (cu_seqlens values, route bits) are
 *     trusted: lengths above max_seqlen are undefined behaviour.
 *   - Functions are thread-safe; the library keeps no state besides the
 *     thread-local last-error text.
 */
#ifndef TILEMIX_H
#define TILEMIX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TILEMIX_OK = 0,
  TILEMIX_ERR_INVALID_ARG = 1,     /* null pointer, bad size, misaligned pointer or stride */
  TILEMIX_ERR_UNSUPPORTED = 2,     /* valid but not implemented (head_dim, block size, causal = 0) */
  TILEMIX_ERR_TOO_MANY_GROUPS = 3, /* ceil(T / g) > 64: a row's groups do not fit one 64-bit word */
  TILEMIX_ERR_WORKSPACE = 4,       /* workspace NULL or smaller than tilemix_attn_workspace_size */
  TILEMIX_ERR_HIP = 5              /* a HIP launch or runtime call failed */
} tilemix_status;

/* Static English name of a status code (never NULL). */
const char* tilemix_status_string(int32_t status);

/* Host: text describing the last failure on the calling thread ("" if none). */
const char* tilemix_last_error(void);

/* Host: library version string. */
const char* tilemix_version(void);

/*
 * Blockwise symmetric INT8 quantisation, quantize-once operand preparation
 * ([PL §3 Preliminaries] blockwise quantisation with INT32 accumulation;
 * [PL App. C] Q8, K8 and block scales made once per attention call).
 *
 * For each head h, sequence b and block k of `blk` consecutive tokens of that
 * sequence (the last block of a sequence may be partial; blocks restart at each
 * sequence start), over all head_dim channels:
 *     a = max |x|;  scale = fl32(a / 127)  (correctly rounded)
 *     q = clamp(round_half_even(fl32(x / scale)), -127, 127)
 * An all-zero block gets scale 1.0f and q = 0.
 *
 *   x          fp16, x[t*stride_tok + h*stride_head + c]; strides in elements,
 *              multiples of 8, x 16-byte aligned, channels contiguous.
 *   x_q        int8 [N][num_heads][head_dim], contiguous (written).
 *   scales     float32 [num_heads][batch][ceil(max_seqlen/blk)] (written);
 *              entries for blocks past a sequence's end are set to 0.
 *   blk        64 or 128 (tokens).  head_dim 64 or 128.
 * Pure device work; bit-exact with the CPU definition above.
 */
int32_t tilemix_quantize_blockwise(const void* x, int64_t stride_tok, int64_t stride_head,
                                   const int32_t* cu_seqlens, int32_t batch, int32_t max_seqlen,
                                   int32_t num_heads, int32_t head_dim, int32_t blk,
                                   int8_t* x_q, float* scales, void* stream);

/*
 * Pack per-tile precision decisions into one 64-bit route word per
 * (KV head, sequence, query-tile row) ([PL §3 Preliminaries], [PL §4],
 * [PL App. D], [AN]).  One bit governs a group of g adjacent key tiles; bit
 * j covers key tiles [j*g, j*g + g) and bit 0 is the least significant.
 *
 *   tile_route  uint8 [num_kv_heads][batch][T][Tk]; nonzero = INT8, 0 = FP16.
 *               Entries of illegal tiles (keys after every query of the row,
 *               or m past the sequence end) are ignored.
 *   cu_seqlens_k, max_seqlen_k: key prefix sums and bound for chunked prefill
 *               (see the conventions above), or NULL and 0 for prefill.
 *   route_words uint64 [num_kv_heads][batch][T] (written).  A group's bit is the
 *               AND of its legal tiles' decisions (FP16 wins when they
 *               disagree); bits of groups with no legal tile and rows past the
 *               sequence end are 0.
 *   g           >= 1 with ceil(Tk/g) <= 64, else TILEMIX_ERR_TOO_MANY_GROUPS.
 */
int32_t tilemix_build_route_mask(const uint8_t* tile_route, const int32_t* cu_seqlens,
                                 const int32_t* cu_seqlens_k, int32_t batch, int32_t max_seqlen,
                                 int32_t max_seqlen_k, int32_t num_kv_heads, int32_t g,
                                 uint64_t* route_words, void* stream);

/*
 * Inverse of the packer, for bit-exact checks: decode R = (word >> floor(n/g)) & 1
 * for every tile ([GS], [PL §3 Preliminaries]).
 *   tile_route_out uint8 [num_kv_heads][batch][T][Tk] (written): legal tiles get
 *                  their bit (1 = INT8), illegal tiles 0xFF.
 */
int32_t tilemix_decode_route_mask(const uint64_t* route_words, const int32_t* cu_seqlens,
                                  const int32_t* cu_seqlens_k, int32_t batch, int32_t max_seqlen,
                                  int32_t max_seqlen_k, int32_t num_kv_heads, int32_t g,
                                  uint8_t* tile_route_out, void* stream);

/* Static routing templates (see tilemix_template_route_words). */
typedef enum {
  TILEMIX_TEMPLATE_ALL_FP16 = 0,
  TILEMIX_TEMPLATE_ALL_INT8 = 1,
  TILEMIX_TEMPLATE_BAND = 2,
  TILEMIX_TEMPLATE_GLOBAL = 3,
  TILEMIX_TEMPLATE_ROW_RANDOM = 4,
  TILEMIX_TEMPLATE_ALIGNED_SPARSE = 5,
  TILEMIX_TEMPLATE_BIGBIRD = 6,
  TILEMIX_TEMPLATE_SPTRANS = 7
} tilemix_template;

/*
 * Route words of a static, data-free routing template at a target INT8 coverage
 * of the legal tile groups ([PL App. B] names the layouts and the coverage
 * settings; [PL Limitations] and [GS]: templates are built once and reused).
 * The pages print no definitions; per query-tile row with n legal groups,
 * F = (( 1000 - int8_permille) * n + 500) / 1000 groups stay FP16, the other legal
 * groups are INT8:
 *   BAND            the F groups nearest the diagonal
 *   GLOBAL          the first F groups
 *   ROW_RANDOM      the F groups with the smallest SplitMix64 keys of
 *                   seed ^ (((hk * batch + b) * T + m) * 64 + j) (ties: lower j)
 *   ALIGNED_SPARSE  the groups floor(k * n / F), k = 0 .. F-1
 *   BIGBIRD         ceil(F/3) band groups, then ceil((F - that)/2) first groups,
 *                   then random groups in key order up to F (an approximation)
 *   SPTRANS         ceil(F/2) band groups, then F - ceil(F/2) groups evenly spaced
 *                   before the band (local + strided; an approximation)
 *   ALL_FP16 / ALL_INT8 ignore int8_permille.
 * Chunked prefill: cu_seqlens_k / max_seqlen_k as for tilemix_build_route_mask.
 *   route_words  uint64 [num_kv_heads][batch][T] (written), bits of illegal groups 0.
 *   int8_permille 0 .. 1000; g >= 1 with ceil(Tk/g) <= 64.
 */
int32_t tilemix_template_route_words(int32_t template_kind, int32_t int8_permille, uint64_t seed,
                                     const int32_t* cu_seqlens, const int32_t* cu_seqlens_k, int32_t batch,
                                     int32_t max_seqlen, int32_t max_seqlen_k, int32_t num_kv_heads,
                                     int32_t g, uint64_t* route_words, void* stream);

/* Host struct: problem description of one attention call. */
typedef struct {
  int32_t batch;        /* sequences, >= 1 */
  int32_t max_seqlen;   /* >= every sequence's query count, >= 1 */
  int32_t num_q_heads;  /* Hq, a multiple of num_kv_heads */
  int32_t num_kv_heads; /* Hk, 1..256 */
  int32_t head_dim;     /* 64 or 128 */
  int32_t g;            /* key tiles per route bit, ceil(T/g) <= 64 */
  int32_t blk_q;        /* Q quantisation block, 64 or 128 tokens; K/V blocks are 64 */
  float sm_scale;       /* softmax scale, > 0 (usually fp32 1/sqrt(head_dim)) */
  int32_t causal;       /* must be 1 */
  int32_t kv_int8;      /* 0: k, v are fp16; 1: k, v are an INT8 cache with scales */
  int32_t out_fp32;     /* 0: out is fp16; 1: out is float32 */
  int32_t otf_quant;    /* 0: quantise-once operands (q_q, q_scale, k_q, k_scale from
                           tilemix_quantize_blockwise); 1: on-the-fly quantisation
                           ([PL App. C], [PL App. D]): the kernel derives the block scales
                           and INT8 fragments of Q and of INT8-routed K tiles on chip from
                           q and k, with the same definition and bit-identical results;
                           q_q, q_scale, k_q and k_scale are not read (may be NULL).
                           2: on-the-fly Q only: Q's block scales and INT8 fragments are
                           made on chip as in 1 (q_q and q_scale are not read), and K
                           takes the quantise-once k_q and k_scale.  Same results as 0
                           and 1, bit for bit; saves the separate pass over Q.
                           1 and 2 require kv_int8 = 0. */
  int32_t max_seqlen_k; /* 0: prefill, the keys are the queries' positions.  > 0: chunked
                           prefill / decode over a KV cache (an extension: the pages scope
                           the method to prefill, [PL Limitations], and list decode as not
                           yet evaluated, [AN], [AF]): >= every key count and
                           >= max_seqlen, with tensors.cu_seqlens_k; K, V, k_q and their
                           scales are packed by cu_seqlens_k, route words index query-tile
                           rows with bits over ceil(max_seqlen_k/64) key tiles. */
} tilemix_attn_params;

/* Host struct of device pointers for one attention call. */
typedef struct {
  const void* q;          /* fp16, q[t*q_stride_tok + h*q_stride_head + c] */
  const void* k;          /* kv_int8 = 0: fp16; 1: int8.  k[t*kv_stride_tok + h*kv_stride_head + c] */
  const void* v;          /* same type and strides as k */
  int64_t q_stride_tok, q_stride_head;    /* elements; multiples of 8; 16-byte aligned base */
  int64_t kv_stride_tok, kv_stride_head;  /* elements; multiples of 8 (fp16) or 16 (int8); 64 rows at
                                             the token stride must span less than 4 GiB (a tile is read
                                             through one 32-bit buffer range), else
                                             TILEMIX_ERR_UNSUPPORTED */
  const int8_t* q_q;      /* int8 [N][Hq][d] contiguous, from tilemix_quantize_blockwise(q, blk_q);
                             unused when otf_quant = 1 or 2 */
  const float* q_scale;   /* float32 [Hq][batch][ceil(max_seqlen/blk_q)]; unused when otf_quant = 1 or 2 */
  const int8_t* k_q;      /* kv_int8 = 0: int8 [N][Hk][d] contiguous (quantize_blockwise(k, 64));
                             unused when kv_int8 = 1 or otf_quant = 1 */
  const float* k_scale;   /* float32 [Hk][batch][Tk]: per 64-token block of K; unused when otf_quant = 1 */
  const float* v_scale;   /* kv_int8 = 1: float32 [Hk][batch][Tk]; 0: unused.  Supported values: 0 (an
                             all-zero block) and [2^-31, 65504/127], the range the quantiser makes from
                             fp16 data; larger values can overflow the fp16 probabilities, smaller ones
                             lose precision in the row sum.  Not checked (device data). */
  const int32_t* cu_seqlens;     /* int32 [batch+1]: queries (and keys, in prefill) */
  const uint64_t* route_words;   /* uint64 [Hk][batch][T] from tilemix_build_route_mask */
  void* out;              /* fp16 or float32 [N][Hq][d] contiguous (written) */
  const int32_t* cu_seqlens_k;   /* int32 [batch+1] key prefix sums when max_seqlen_k > 0, else NULL */
  float* lse;             /* optional (NULL = not written): float32 [N][Hq], natural-log
                             log-sum-exp of each query row's scores s_ij, for merging
                             partial attentions */
} tilemix_attn_tensors;

/* Host: bytes of device workspace tilemix_attn_prefill needs for `params`. */
int32_t tilemix_attn_workspace_size(const tilemix_attn_params* params, size_t* bytes);

/*
 * Fused causal routed prefill attention ([PL §1], [PL §3 Preliminaries],
 * [PL §4], [PL App. C], [AN]).
 *
 * For every sequence b, query head hq (KV head hk = hq / (Hq/Hk): contiguous
 * GQA groups share K/V and route words, [PL §4]) and query tile m, the legal key
 * tiles n = 0..m are streamed in order.  Route bit R = (route_words[hk][b][m] >>
 * floor(n/g)) & 1 selects the score path of tile (m, n):
 *   R = 0 (FP16):  s_ij = sm_scale * sum_c q_ic k_jc   (fp16 MFMA, fp32 accumulation;
 *                  kv_int8 = 1 uses k = k_int8 * k_scale exactly)
 *   R = 1 (INT8):  s_ij = sm_scale * q_scale(i) * k_scale(j) * S32_ij,
 *                  S32 = int8 MFMA with exact int32 accumulation of q_q . k_q
 *                  (otf_quant = 1: q_q, k_q and their scales are made on chip;
 *                  otf_quant = 2: q_q and q_scale)
 * Both paths update one online-softmax state per query row (running max, sum
 * and output accumulator in fp32); P.V runs in fp16 with fp32 accumulation
 * (kv_int8 = 1: v = v_int8 * v_scale, the scale folded into P); the output is
 * acc / sum.  Key j is legal for query i iff j <= i < L_b (top-left causal), or
 * with cu_seqlens_k iff j <= (Lk_b - Lq_b) + i (chunked prefill; decode is Lq_b = 1).
 *
 * `workspace` must hold tilemix_attn_workspace_size() bytes (256-byte aligned);
 * it receives the varlen/GQA work list, rebuilt on every call.  Equivalent to
 * tilemix_attn_plan followed by tilemix_attn_run on the same stream.
 */
int32_t tilemix_attn_prefill(const tilemix_attn_params* params, const tilemix_attn_tensors* tensors,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the device array that holds tilemix_attn_prefill_noalloc's work list. */
#define TILEMIX_NOALLOC_WORKSPACE_BYTES (4u << 20)

/*
 * tilemix_attn_prefill without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same computation, kernels and output bits
 * as tilemix_attn_prefill; the work list goes to a file-scope device array of
 * TILEMIX_NOALLOC_WORKSPACE_BYTES (4 MiB) that the library holds on every GPU
 * it runs on until the process ends.  The call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine).
 *
 * Limit: calls whose work list (tilemix_attn_workspace_size) exceeds the array
 * are rejected with TILEMIX_ERR_WORKSPACE before any launch.  4 MiB holds
 * about 250,000 work items (16 bytes each, plus a segment table): batch 480 of
 * 4096 tokens with 8 KV heads and 3 query heads per KV head (245,760 items)
 * fits; the 3B-shaped batch of 8 needs 4,096.
 * Device and concurrency: the array of the current device is used (take the
 * stream from that device).  Every call on one GPU shares its array and rewrites
 * the whole work list before reading it, so calls that overlap on one GPU
 * (several streams or threads at once) race; serialise them.
 * Errors: as tilemix_attn_prefill, plus TILEMIX_ERR_HIP if the array's device
 * address cannot be obtained.
 */
int32_t tilemix_attn_prefill_noalloc(const tilemix_attn_params* params, const tilemix_attn_tensors* tensors,
                                     void* stream);

/*
 * The varlen/GQA work schedule alone ([PL §4]: prefix-sum metadata,
 * padding-free execution): from cu_seqlens (device int32 [batch+1]; with
 * cu_seqlens_k for chunked prefill, NULL otherwise, as in the tensors) it writes
 * the work list of (sequence, KV head, query tile, head chunk) items into
 * `workspace`, longest causal rows first, each (sequence, KV head) group kept
 * on one XCD where the slots allow.  Asynchronous on `stream`; no allocation.
 * The list depends only on `params` and cu_seqlens, so several layers of one
 * batch may share it.
 */
int32_t tilemix_attn_plan(const tilemix_attn_params* params, const int32_t* cu_seqlens,
                          const int32_t* cu_seqlens_k, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The attention of tilemix_attn_prefill over the work list a previous
 * tilemix_attn_plan wrote into `workspace` (same params, same cu_seqlens
 * contents, ordered before this call on the stream).  Items whose indices fall
 * outside the problem are skipped, so a stale or missing list gives wrong
 * output, never an out-of-range access.
 */
int32_t tilemix_attn_run(const tilemix_attn_params* params, const tilemix_attn_tensors* tensors, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Host struct: debug products of tilemix_attn_prefill_debug (device pointers, any may be NULL). */
typedef struct {
  int32_t seq, q_head, m_begin, m_end;  /* window of query-tile rows whose INT32 tiles are dumped */
  int32_t* s32_tiles;      /* int32 [m_end-m_begin][Tk][64][64] (query offset, key offset):
                              raw INT32 score tile of every INT8-routed tile; others INT32_MIN */
  uint32_t* visit_count;   /* uint32 [batch][Hq][T][Tk]: +1 per tile visit (zeroed by the call) */
  uint8_t* route_used;     /* uint8 [batch][Hq][T][Tk]: path taken, 0xFF if not visited */
} tilemix_debug;

/* Same computation and output as tilemix_attn_prefill, plus the debug products
 * (for bit-exact checks of the INT32 scores, tile coverage and decoded routes). */
int32_t tilemix_attn_prefill_debug(const tilemix_attn_params* params, const tilemix_attn_tensors* tensors,
                                   void* workspace, size_t workspace_bytes, const tilemix_debug* dbg,
                                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TILEMIX_H */
